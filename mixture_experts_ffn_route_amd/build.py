"""Ahead-of-time build of the gfx950 HIP library ``libmoe_mi355x.so`` (in-tree).

``python mixture_experts_ffn_route_amd/build.py`` compiles every source under
``csrc/`` with hipcc for gfx950 and links the shared library next to this
file.  Objects go to ``_build/`` at the repository root.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# The same library with the 256-token GEMM's slot timers compiled in
# (moe_debug_slot_timers); loaded instead of LIB_NAME when MOE_SLOT_TIMERS=1.
TIMERS_LIB_NAME = "libmoe_mi355x_slot_timers.so"
TIMERS_LIB_PATH = os.path.join(PKG, TIMERS_LIB_NAME)
ARCH = "gfx950"

SOURCES = [
    "moe_host.cpp",
    "moe_api.cpp",
    "moe_stage.hip",
    "moe_compact.hip",
    "moe_gemm_fp8.hip",
    "moe_gemm_mx.hip",
    "moe_swiglu.hip",
    "moe_combine.hip",
    "moe_weights.hip",
    "moe_noalloc.hip",
]

# Packed FP32 VALU ops are disabled for all device code.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    warn = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip())
    if warn and verbose:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False, slot_timers: bool = False) -> str:
    """Compile and link; returns the library path.  Always rebuilds.
    slot_timers: build the timed variant (TIMERS_LIB_NAME) instead."""
    build_dir = os.path.join(BUILD, "slot_timers") if slot_timers else BUILD
    extra = ("-DMOE_SLOT_TIMERS=1",) if slot_timers else ()
    out = TIMERS_LIB_PATH if slot_timers else LIB_PATH
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, slot_timers="--slot-timers" in sys.argv))
