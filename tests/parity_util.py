"""Comparison rules between the HIP path and the oracle.

Integer and index results (routing, counts, offsets, compaction indices,
staged codes) are compared bit for bit.  The BF16 layer output must have a
relative Frobenius error <= 1e-2 and at least 99.9% of its elements within
5e-2 of their row's RMS (this leaves room for the occasional e4m3
requantisation flip, and for FP32 accumulation on the GPU against float64 in
the oracle).
"""

import numpy as np

REL_FROB = 1e-2
ELEM_FRAC = 0.999
ELEM_TOL = 5e-2


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def output_error(got_bits, want_bits):
    g = bf16_bits_to_f64(got_bits)
    w = bf16_bits_to_f64(want_bits)
    assert g.shape == w.shape
    assert np.all(np.isfinite(g)), "non-finite output"
    den = np.linalg.norm(w)
    rel = np.linalg.norm(g - w) / den if den > 0 else np.linalg.norm(g)
    rms = np.sqrt(np.mean(w * w, axis=1, keepdims=True))
    ok = np.abs(g - w) <= ELEM_TOL * rms
    zero_rows = (rms[:, 0] == 0)
    frac = ok[~zero_rows].mean() if (~zero_rows).any() else 1.0
    return rel, frac, g, w, zero_rows


def assert_output_close(got_bits, want_bits, label=""):
    rel, frac, g, w, zero_rows = output_error(got_bits, want_bits)
    assert rel <= REL_FROB, f"{label}: relative Frobenius error {rel:.3e} > {REL_FROB}"
    assert frac >= ELEM_FRAC, f"{label}: only {frac:.5f} of elements within {ELEM_TOL} x row RMS"
    # rows the oracle leaves at +0 (every route masked) must be exactly +0
    assert np.all(np.asarray(got_bits)[zero_rows] == 0), f"{label}: masked token rows are not +0"
    return rel, frac


# The FP8 GEMM's FP32 output (gate/up before SwiGLU) against the float64
# product of its dequantised operands.  Per output, K-block kb adds the
# MFMA's sum of 128 e4m3 products times the block's scale product F_kb; the
# MFMA's error is at most 2^-10 of its largest product (measured:
# test_gpu_mfma_accumulation), bounded here by the block maxima of |x| and
# |w|; the promotion multiply, the MFMA's addition of the running
# accumulator and the final multiply each round once more to FP32, at most
# (kbs + 2) * 2^-24 * sum_k |x_k w_k| in all.
MFMA_BETA = 2.0 ** -10


def gemm_error_bound(x_rows, w_rows):
    """Elementwise bound on |FP32 GEMM - exact| for x_rows [n, K] @ w_rows[m, K]^T
    (dequantised float64 operands, K a multiple of 128)."""
    n, K = x_rows.shape
    kbs = K // 128
    ax = np.abs(x_rows).reshape(n, kbs, 128).max(axis=2)
    aw = np.abs(w_rows).reshape(w_rows.shape[0], kbs, 128).max(axis=2)
    return MFMA_BETA * (ax @ aw.T) + (kbs + 2) * 2.0 ** -24 * (np.abs(x_rows) @ np.abs(w_rows).T)
