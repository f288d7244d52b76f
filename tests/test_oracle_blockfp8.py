"""Pins of the block-FP8 (128 x 128) oracle (oracle/blockfp8.py) against things other
than itself: numpy's and torch's float32 division and float8_e4m3fn cast (library
routines), the format's own bounds, and an exact loop model of the layer on a tiny
shape (tests/brute_force.py, exact rationals and torch casts)."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import blockfp8 as B
from oracle import codecs as C
from tests import brute_force as BF


def _bf16(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return W.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_block_scale_is_amax_over_448_in_float32():
    w = _bf16((2, 256, 384), 1, 0.02)
    codes, s = B.quant_weights(w)
    v = C.bf16_value(w).astype(np.float32).reshape(2, 2, 128, 3, 128)
    amax = np.abs(v).max(axis=(2, 4))
    assert s.dtype == np.float32 and s.shape == (2, 2, 3)
    assert np.array_equal(s, amax / np.float32(448.0))          # numpy's float32 division


def test_codes_match_torch_float8_cast():
    w = _bf16((256, 256), 2, 0.02)
    codes, s = B.quant_weights(w)
    v = torch.from_numpy(C.bf16_value(w).astype(np.float32)).reshape(2, 128, 2, 128)
    st = torch.from_numpy(s)[:, None, :, None]
    q = torch.clamp(v / st, -448.0, 448.0)                      # torch's float32 division
    ref = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(256, 256).numpy()
    assert np.array_equal(codes, ref)


def test_largest_element_of_each_block_maps_to_448():
    x = _bf16((5, 512), 3)
    codes, s = B.quant_act(x)
    v = C.bf16_value(x).astype(np.float32).reshape(5, 4, 128)
    c = codes.reshape(5, 4, 128)
    arg = np.abs(v).argmax(axis=-1)
    top = np.take_along_axis(c, arg[..., None], -1)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)                          # |code value| = 448


def test_quantisation_error_is_at_most_half_a_step():
    x = _bf16((7, 1024), 4, 3.0)
    codes, s = B.quant_act(x)
    v = C.bf16_value(x).astype(np.float64)
    dq = B.dequant_rows(codes, s)
    sc = np.repeat(s.astype(np.float64), 128, -1)
    # normal E4M3 values: half a step is at most 2^-4 of the magnitude; subnormals
    # (|v/s| < 2^-6): half of 2^-9; plus the float32 rounding of v/s
    lim = np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * sc) * (1 + 2.0 ** -20) + 2.0 ** -24 * np.abs(v)
    assert np.all(np.abs(dq - v) <= lim)


def test_zero_block_has_unit_scale_and_zero_codes():
    x = np.zeros((2, 256), np.uint16)
    x[1, 128:] = _bf16((1, 128), 5)[0]
    codes, s = B.quant_act(x)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert not codes[0].any() and not codes[1, :128].any()


SHAPE = W.Workload("fp8b_tiny", T=3, H=128, I=128, E=2, topk=2)


def _tiny_inputs():
    w = SHAPE
    x = W.gen_x(w)
    logits = W.gen_logits(w)
    w13 = np.stack([W.gen_expert_w13(w, e) for e in range(w.E)])
    w2 = np.stack([W.gen_expert_w2(w, e) for e in range(w.E)])
    return x, logits, w13, w2


def _compare_with_brute():
    w = SHAPE
    x, logits, w13, w2 = _tiny_inputs()
    q13, s13 = B.quant_weights(w13)
    q2, s2 = B.quant_weights(w2)
    got = B.forward(x, q13, s13, q2, s2, topk=w.topk, I=w.I, logits=logits)
    ref = BF.layer_fp8b(x, w13, w2, w.topk, w.I, logits)
    assert np.array_equal(got["topk_idx"], np.array(ref["idx"]))
    so = got["slot_of"]
    for (t, j), (hc, hs) in ref["hq"].items():
        p = so[t, j]
        assert np.array_equal(got["hq"][p], np.array(hc, np.uint8)), (t, j)
        assert np.array_equal(got["hsf"][p], np.array(hs, np.float32)), (t, j)
    a = C.bf16_value(got["y"]).astype(np.float64)
    b = C.bf16_value(np.array(ref["y"], np.uint16)).astype(np.float64)
    # the same computation up to the float64 rounding of 56-bit products (about 2^-45
    # relative), which can move a BF16 rounding decision by one BF16 step
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-30)
    assert np.mean(a == b) >= 0.99


@pytest.mark.slow
def test_layer_matches_exact_loop_model():
    _compare_with_brute()
