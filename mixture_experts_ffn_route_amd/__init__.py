"""MI355X-native MegaMoE per-rank layer forward.

The compute path lives in the HIP library ``libmoe_mi355x.so`` (C ABI in
``include/moe.h``); ``_lib`` binds it with ctypes and ``layer.MoELayer``
owns one handle with torch-allocated device memory.  Importing the package
fails if the library has not been built.
"""

from . import _lib  # noqa: F401  (raises ImportError if the library is missing)
from ._lib import MoEError  # noqa: F401
from .layer import MoELayer  # noqa: F401
