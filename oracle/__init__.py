"""CPU oracle for the MegaMoE per-rank layer forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy statement of what the layer computes, used to
check the HIP path.  Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library itself never
calls it and shares no code, header, table or helper with it.

Sources (pages of the flashinfer ``moe_ep`` pull-request series):

* "feat(moe_ep): add SM90 push FP8 mega-MoE backend for Hopper" (PR #4069):
  Description (the forward pipeline: compact -> FC1 with fused SwiGLU + 1x128
  quantisation -> FC2 -> grouped combine with owner-side FP32 route
  reduction), its bullet list (dedup dispatch, grouped combine, fused FC1
  epilogue) and Limitations (top_k set, DeepSeek-style FP8 block scaling,
  SwiGLU only).
* "perf(moe_ep): fuse Rubin MegaMoE forward preparation" (PR #6398):
  Description and its follow-up commit (input quantisation + route staging,
  route checker semantics, masked routes with non-finite scores).
* "feat(moe_ep): MXFP8 x BF16 integration" (PR #4604): Description (BF16
  activations x MXFP8 weights, BF16 output, MXFP8 decode + BF16 reference).

Parity status per function is listed in ``oracle.moe_ref.PIN_STATUS``.
"""

from . import formats, moe_ref  # noqa: F401
