"""Pins of the workload shapes and quantisation layouts to sizes the pages print
(tests/golden/pages_shapes.json, each entry with its page and section)."""
import json
import os

import numpy as np

import moe_workloads as W
from oracle import moe_ref as M

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.json")))


def test_dsv3_shapes_match_scheduler_example():
    g = GOLD["dsv3_scheduler_example"]
    for name in ("dsv3_prefill", "dsv3_skewed"):
        w = W.WORKLOADS[name]
        assert 2 * w.I == g["l1_n"] and w.H == g["l2_n"]
        # the example's per-expert N-block counts at BLOCK_N = 128
        assert 2 * w.I // g["block_n"] == g["l1_blocks_n"]
        assert w.H // g["block_n"] == g["l2_blocks_n"]


def test_decode_shape_matches_fixed_shape():
    g = GOLD["decode_fixed_shape"]
    w = W.WORKLOADS["decode"]
    assert (w.E, w.H, w.I) == (g["experts"], g["hidden"], g["n_per_projection"])
    assert w.T <= g["max_tokens"]


def test_weight_quantisation_shapes():
    g = GOLD["weight_quantisation"]
    G, n, k = 2, 8, 4 * g["group"]
    w = W.to_bf16_bits(np.random.default_rng(0).standard_normal((G, n, k)).astype(np.float32))
    q, sf = M.pack_weights(w)
    assert sf.shape == (G, n, k // g["group"]) and sf.dtype == np.uint8
    assert q.shape == (G, n, k // 2)            # k FP4 codes, two per byte


def test_activation_quantisation_groups_along_hidden():
    g = GOLD["activation_quantisation"]
    x = W.to_bf16_bits(np.random.default_rng(1).standard_normal((3, 4 * g["group"])).astype(np.float32))
    q, sf = M.quant_act(x)
    assert q.shape == x.shape and sf.shape == (3, 4)
    # one scale per 32 consecutive hidden elements: scaling one group changes only its scale
    x2 = x.copy()
    v = W.bf16_bits_to_f32(x2[1, 32:64]) * np.float32(4.0)
    x2[1, 32:64] = W.to_bf16_bits(v)
    q2, sf2 = M.quant_act(x2)
    changed = sf2 != sf
    assert changed[1, 1] and changed.sum() == 1 and sf2[1, 1] == sf[1, 1] + 2
    assert np.array_equal(q2, q)
