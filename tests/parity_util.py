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
