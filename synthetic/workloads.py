"""Seeded synthetic inputs with the shapes and value distributions of the
MegaMoE per-rank layer workloads.

Recipe (every stream is an independent ``numpy.random.Generator(PCG64)``
seeded from ``SeedSequence([seed, stream, index])``, so any expert's weights
can be regenerated alone):

* router logits ``~N(0, 1)`` of shape ``[T, E]`` (stream ``ROUTER``), then one
  of three routing rules (``make_routing``);
* activations ``x ~ N(0, 1)`` drawn in float32 and rounded to bfloat16 by
  torch's cast (stream ``X``);
* FC1 weights ``W13[e] ~ N(0, 1/H)`` of shape ``[2I, H]`` -- the first ``I``
  rows are the gate projection, the next ``I`` rows the up projection -- and
  FC2 weights ``W2[e] ~ N(0, 1/H)`` of shape ``[H, I]`` (streams ``W13``,
  ``W2``, one sub-stream per expert);
* weights stored either as e4m3 codes with one float32 scale per 128x128 block
  (scale = amax/448, the DeepSeek-style block scaling the SM90 push backend
  page lists among its supported configurations), or as e4m3 or e5m2 codes
  with one E8M0 exponent per 32 consecutive K elements (the OCP MX v1.0 rule
  used by the MXFP8 x BF16 MegaMoE integration page).

The float8 encodings are done by torch's ``float8_e4m3fn`` / ``float8_e5m2``
casts after clamping to the format's largest finite value; nothing here
re-implements the layer's quantisers.
"""

from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np
import torch

# Stream identifiers (fixed draw order: router logits, x, W13, W2).
ROUTER, X, W13, W2, MASK = 1, 2, 3, 4, 5

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


@dataclass(frozen=True)
class MoEShape:
    tokens: int
    hidden: int
    intermediate: int
    experts: int
    top_k: int
    routing: str = "topk"  # "topk" | "balanced" | "zipf"

    @property
    def routes(self) -> int:
        return self.tokens * self.top_k


# Workload shapes.  "dsv3" is one GPU's share of a DeepSeek-V3-like layer
# (256 experts over 8 GPUs -> 32 local experts).
CONFIGS: Dict[str, MoEShape] = {
    "tiny": MoEShape(16, 256, 128, 8, 2, "topk"),
    "small": MoEShape(512, 2048, 768, 32, 6, "topk"),
    "dsv3": MoEShape(4096, 7168, 2048, 32, 8, "balanced"),
    "skewed": MoEShape(8192, 7168, 2048, 32, 8, "zipf"),
}
SWEEP_TOKENS = (8, 64, 512, 4096, 32768)


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, index])))


def _softmax64(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=-1, keepdims=True)


def token_groups_balanced(tokens: int, experts: int, top_k: int, rng: np.random.Generator) -> np.ndarray:
    """Block-permutation balanced assignment.

    Tokens are taken in groups of ``experts // top_k``; each group draws one
    random permutation of the experts and token ``j`` of the group takes the
    ``j``-th run of ``top_k`` entries.  With ``experts % top_k == 0`` and
    ``tokens`` a multiple of the group size every expert receives exactly
    ``tokens * top_k / experts`` routes.
    """
    group = max(1, experts // top_k)
    idx = np.empty((tokens, top_k), dtype=np.int64)
    for g0 in range(0, tokens, group):
        perm = rng.permutation(experts)
        for j in range(min(group, tokens - g0)):
            idx[g0 + j] = perm[j * top_k:(j + 1) * top_k]
    return idx


def make_routing(shape: MoEShape, seed: int = 0, masked_fraction: float = 0.0,
                 zero_experts: int = 4, zipf_s: float = 1.2) -> Tuple[np.ndarray, np.ndarray]:
    """Return ``(topk_idx int32 [T, K], topk_w float32 [T, K])``.

    * ``topk``: softmax over all E logits in float64, the K most probable
      experts (ties to the lower id), slots in descending probability, weights
      renormalised over the K chosen experts.
    * ``balanced``: block-permutation assignment (``token_groups_balanced``),
      weights = softmax of the token's logits restricted to its experts.
    * ``zipf``: ``zero_experts`` experts receive nothing; the rest get
      popularity ``p ~ rank^-zipf_s`` over a random rank order; each token
      samples K distinct experts by Gumbel-top-k on ``log p``.  Weights as in
      ``balanced``.

    ``masked_fraction > 0`` replaces that fraction of slots with expert -1
    carrying NaN/+inf/-inf weights (masked routes), and masks every slot of the
    last token.
    """
    T, E, K = shape.tokens, shape.experts, shape.top_k
    rng = _rng(seed, ROUTER)
    logits = rng.standard_normal((T, E))
    if shape.routing == "topk":
        p = _softmax64(logits)
        order = np.argsort(-p, axis=1, kind="stable")[:, :K]
        idx = order
    elif shape.routing == "balanced":
        idx = token_groups_balanced(T, E, K, rng)
    elif shape.routing == "zipf":
        zero = rng.choice(E, size=min(zero_experts, E - K), replace=False)
        active = np.setdiff1d(np.arange(E), zero)
        ranks = rng.permutation(active.size) + 1
        logp = np.full(E, -np.inf)
        logp[active] = -zipf_s * np.log(ranks.astype(np.float64))
        gumbel = rng.gumbel(size=(T, E))
        keys = logp[None, :] + gumbel
        idx = np.argsort(-keys, axis=1, kind="stable")[:, :K]
    else:
        raise ValueError(f"unknown routing {shape.routing!r}")
    sel = np.take_along_axis(logits, idx, axis=1)
    w = _softmax64(sel).astype(np.float32)
    idx = idx.astype(np.int32)
    if masked_fraction > 0.0:
        mrng = _rng(seed, MASK)
        m = mrng.random((T, K)) < masked_fraction
        m[-1, :] = True
        idx = np.where(m, np.int32(-1), idx)
        junk = np.array([np.nan, np.inf, -np.inf], dtype=np.float32)
        w = np.where(m, junk[mrng.integers(0, 3, size=(T, K))], w).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


def make_activations(tokens: int, hidden: int, seed: int = 0) -> np.ndarray:
    """x ~ N(0, 1) rounded to bfloat16; returned as raw uint16 bit patterns."""
    z = _rng(seed, X).standard_normal((tokens, hidden), dtype=np.float32)
    return torch.from_numpy(z).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_weights(seed: int, stream: int, e: int, rows: int, cols: int, hidden: int) -> np.ndarray:
    z = _rng(seed, stream, e).standard_normal((rows, cols), dtype=np.float32)
    return z * np.float32(1.0 / math.sqrt(hidden))


def _e4m3_codes(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v, -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _block_quant_one(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    n, k = w.shape
    blk = w.reshape(n // 128, 128, k // 128, 128)
    amax = np.abs(blk).max(axis=(1, 3))
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0))
    v = blk / safe[:, None, :, None]
    v = np.where((scale > 0)[:, None, :, None], v, np.float32(0.0))
    return _e4m3_codes(v.reshape(n, k)), scale


def _e5m2_codes(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v, -E5M2_MAX, E5M2_MAX))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def _mx_quant_one(w: np.ndarray, elem: str = "e4m3") -> Tuple[np.ndarray, np.ndarray]:
    """OCP MX v1.0: shared exponent floor(log2 amax_32) - emax(elem), elements
    cast to the element type (emax 8 for e4m3, 15 for e5m2)."""
    n, k = w.shape
    blk = w.reshape(n, k // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)  # amax = m * 2**ex, m in [0.5, 1)
    emax = 15 if elem == "e5m2" else 8
    shared = np.where(amax > 0, ex.astype(np.int32) - 1 - emax, -127)
    shared = np.clip(shared, -127, 127).astype(np.int32)
    v = np.ldexp(blk, -shared[:, :, None]).astype(np.float32)
    codes = _e5m2_codes(v.reshape(n, k)) if elem == "e5m2" else _e4m3_codes(v.reshape(n, k))
    return codes, (shared + 127).astype(np.uint8)


def _mx_quant_one_e5m2(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    return _mx_quant_one(w, "e5m2")


def _per_expert(fn, seed, stream, experts, rows, cols, hidden):
    def one(e):
        return fn(_normal_weights(seed, stream, e, rows, cols, hidden))

    if experts * rows * cols <= (1 << 22):
        parts = [one(e) for e in range(experts)]
    else:
        with _cf.ThreadPoolExecutor(max_workers=_workers()) as ex:
            parts = list(ex.map(one, range(experts)))
    codes = np.stack([p[0] for p in parts])
    scales = np.stack([p[1] for p in parts])
    return codes, scales


def make_fp8_block_weights(experts: int, rows: int, cols: int, hidden: int, seed: int, stream: int):
    """e4m3 codes ``uint8 [E, rows, cols]`` + float32 scales ``[E, rows/128, cols/128]``."""
    return _per_expert(_block_quant_one, seed, stream, experts, rows, cols, hidden)


def make_mxfp8_weights(experts: int, rows: int, cols: int, hidden: int, seed: int, stream: int,
                       elem: str = "e4m3"):
    """e4m3 (or e5m2) codes ``uint8 [E, rows, cols]`` + E8M0 exponents ``uint8 [E, rows, cols/32]``."""
    fn = _mx_quant_one_e5m2 if elem == "e5m2" else _mx_quant_one
    return _per_expert(fn, seed, stream, experts, rows, cols, hidden)


@dataclass
class LayerInputs:
    shape: MoEShape
    weight_format: str  # "fp8_block" | "mxfp8" | "mxfp8_e5m2"
    x_bf16: np.ndarray  # uint16 [T, H]
    topk_idx: np.ndarray  # int32 [T, K]
    topk_w: np.ndarray  # float32 [T, K]
    w13: np.ndarray  # uint8 [E, 2I, H]
    w13_scale: np.ndarray  # float32 [E, 2I/128, H/128] or uint8 [E, 2I, H/32]
    w2: np.ndarray  # uint8 [E, H, I]
    w2_scale: np.ndarray  # float32 [E, H/128, I/128] or uint8 [E, H, I/32]
    extra: dict = field(default_factory=dict)


def make_layer_inputs(shape: MoEShape, seed: int = 0, weight_format: str = "fp8_block",
                      masked_fraction: float = 0.0, tokens: Optional[int] = None) -> LayerInputs:
    if tokens is not None:
        shape = MoEShape(tokens, shape.hidden, shape.intermediate, shape.experts, shape.top_k, shape.routing)
    T, H, I, E = shape.tokens, shape.hidden, shape.intermediate, shape.experts
    idx, w = make_routing(shape, seed, masked_fraction=masked_fraction)
    x = make_activations(T, H, seed)
    if weight_format not in ("fp8_block", "mxfp8", "mxfp8_e5m2"):
        raise ValueError(weight_format)
    if weight_format == "fp8_block":
        maker = make_fp8_block_weights
    else:
        elem = "e5m2" if weight_format == "mxfp8_e5m2" else "e4m3"
        maker = lambda *a: make_mxfp8_weights(*a, elem=elem)  # noqa: E731
    w13, s13 = maker(E, 2 * I, H, H, seed, W13)
    w2, s2 = maker(E, H, I, H, seed, W2)
    return LayerInputs(shape, weight_format, x, idx, w, w13, s13, w2, s2)
