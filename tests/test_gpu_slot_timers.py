"""The 256-token GEMM's slot timers (library built with build.py
--slot-timers, loaded with MOE_SLOT_TIMERS=1): a forward in a child process
counts exactly one K-block per wave, tile and K-block of each GEMM, every
phase counter moves, and the output equals the plain library's bit for bit
(the counter reads change no arithmetic)."""

import dataclasses
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from mixture_experts_ffn_route_amd import _lib as L
from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device
from synthetic import CONFIGS, make_layer_inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TIMED_LIB = os.path.join(ROOT, "mixture_experts_ffn_route_amd", "libmoe_mi355x_slot_timers.so")

# small config (H=2048, I=768, E=32, K=6) at T=4096: 768 routes per expert,
# 256-token tiles; FC1 16 K-blocks x 6 column tiles, FC2 6 K-blocks x 8
CHILD = r"""
import dataclasses, json, os, sys
sys.path.insert(0, os.getcwd())
import numpy as np, torch
from mixture_experts_ffn_route_amd import _lib as L
from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device
from synthetic import CONFIGS, make_layer_inputs
assert L.SLOT_TIMERS and L.LIB_PATH.endswith("libmoe_mi355x_slot_timers.so")
shape = dataclasses.replace(CONFIGS["small"], tokens=4096)
inp = make_layer_inputs(shape, seed=7)
dev = to_device(inp)
layer = make_layer(shape, dev)
L.moe_debug_slot_timers()
out = run_forward(layer, dev)
torch.cuda.synchronize()
words = L.moe_debug_slot_timers()
np.save(sys.argv[1], out.view(torch.int16).cpu().numpy())
print(json.dumps({"words": words, "block_m": layer.tactic()["block_m"], "status": layer.status()}))
"""


def test_slot_timers_count_every_k_block(tmp_path):
    if not os.path.exists(TIMED_LIB):
        pytest.skip("the slot-timer library is not built (build.py --slot-timers)")
    print("slot timers: small config, T=4096, child process", flush=True)
    out_path = str(tmp_path / "timed_out.npy")
    env = dict(os.environ, MOE_SLOT_TIMERS="1")
    r = subprocess.run([sys.executable, "-c", CHILD, out_path], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    rep = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])
    assert rep["status"] == 0 and rep["block_m"] == 256
    w = rep["words"]
    assert len(w) == L.MOE_SLOT_TIMER_WORDS

    shape = dataclasses.replace(CONFIGS["small"], tokens=4096)
    inp = make_layer_inputs(shape, seed=7)
    idx = inp.topk_idx.reshape(-1)
    n_e = np.bincount(idx[idx >= 0], minlength=shape.experts)
    m_tiles = int(np.sum((n_e + 255) // 256))
    expect = {0: m_tiles * (shape.intermediate // 128) * (shape.hidden // 128) * 4,   # FC1
              16: m_tiles * (shape.hidden // 256) * (shape.intermediate // 128) * 4}  # FC2
    for base, k_blocks in expect.items():
        for grp in range(2):
            d = w[base + grp * 8: base + grp * 8 + 8]
            assert d[7] == k_blocks, (base, grp, d[7], k_blocks)
            # DMA issue, load-slot reads, MFMA issue and epilogue always take time
            for i in (0, 1, 3, 6):
                assert d[i] > 0, (base, grp, i)

    # the same forward on the plain library: identical output bits
    dev = to_device(inp)
    layer = make_layer(shape, dev)
    ref = run_forward(layer, dev).view(torch.int16).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(np.load(out_path), ref)
