"""Planted mistakes in the oracle must be caught by its pins.

Each case patches one plausible error into oracle code (on the CPU only) and
runs the pin that should notice it; the pin must fail.
"""
import numpy as np
import pytest

import moe_workloads as W
from oracle import codecs as C
from oracle import moe_ref as M
from tests import test_oracle_codecs as TC
from tests import test_oracle_layer as TL

SMALL = W.Workload("mut", T=3, H=32, I=32, E=2, topk=2)


_ORIG_SILU = M.silu_mul_weight
_ORIG_EXPERT_ROWS = M.expert_rows


def _swapped_gate_up(g, u, w):
    return _ORIG_SILU(u, g, w)


def _dropped_weight(g, u, w):
    return _ORIG_SILU(g, u, np.ones_like(w))


def _no_silu(g, u, w):
    return (np.asarray(g, np.float64) * u * w).astype(np.float32)


def _transposed_w2(xq_rows, xsf_rows, wts, w13q, w13sf, w2q, w2sf, I):
    # uses W2 as if stored [I, H] (a transposed operand); shapes agree when H == I
    codes = C.unpack_e2m1(w2q)
    sf = np.repeat(w2sf, 32, axis=1)
    w2t_codes = codes.T.copy()
    hq, hsf, acc1, _ = _ORIG_EXPERT_ROWS(xq_rows, xsf_rows, wts, w13q, w13sf, w2q, w2sf, I)
    a2 = C.dequantize_blocks(hq, hsf, "e4m3")
    b2 = C.E2M1_TABLE[w2t_codes.astype(int)] * C.e8m0_value(sf.T)
    return hq, hsf, acc1, C.bf16_bits((a2 @ b2.T).astype(np.float32))


def _run_layer_pin():
    TL._compare_with_brute(SMALL)


@pytest.mark.parametrize("patch", [_swapped_gate_up, _dropped_weight, _no_silu],
                         ids=["swapped_gate_up", "dropped_topk_weight", "missing_silu"])
def test_epilogue_mistakes_are_caught(monkeypatch, patch):
    monkeypatch.setattr(M, "silu_mul_weight", patch)
    with pytest.raises(AssertionError):
        _run_layer_pin()


def test_transposed_gemm2_operand_is_caught(monkeypatch):
    monkeypatch.setattr(M, "expert_rows", _transposed_w2)
    with pytest.raises(AssertionError):
        _run_layer_pin()


def test_off_by_one_block_exponent_is_caught(monkeypatch):
    orig = C.block_exponent
    monkeypatch.setattr(C, "block_exponent", lambda a, q: np.clip(orig(a, q) + 1, -127, 127))
    with pytest.raises(AssertionError):
        TC.test_quantiser_scale_is_minimal("e4m3", 448.0)


def test_ties_away_from_zero_is_caught(monkeypatch):
    def away(x, grid):
        x = np.asarray(x, np.float64)
        hi = np.clip(np.searchsorted(grid, x, side="left"), 1, len(grid) - 1)
        lo = hi - 1
        mid = (grid[lo] + grid[hi]) / 2
        code = np.where(x < mid, lo, hi)
        code = np.where(x >= grid[-1], len(grid) - 1, code)
        return code.astype(np.uint8)
    monkeypatch.setattr(C, "_nearest_even", away)
    with pytest.raises(AssertionError):
        TC.test_e4m3_encode_matches_torch_random_fp32()


def test_ties_to_higher_expert_is_caught(monkeypatch):
    orig = M.route

    def route_hi(logits, topk, score_fn=M.SOFTMAX, renorm=True):
        l = np.asarray(logits, np.float32)[:, ::-1]
        idx, w = orig(l, topk, score_fn, renorm)
        return (l.shape[1] - 1 - idx).astype(np.int32), w
    monkeypatch.setattr(M, "route", route_hi)
    with pytest.raises(AssertionError):
        TL.test_route_matches_sort_based_brute_force(M.SOFTMAX, True)


def test_inclusive_prefix_sum_is_caught(monkeypatch):
    orig = M.bucketize

    def bad(topk_idx, E):
        counts, offsets, slot_src, slot_of = orig(topk_idx, E)
        return counts, np.concatenate([np.cumsum(counts), [offsets[-1]]]).astype(np.int32), slot_src, slot_of
    monkeypatch.setattr(M, "bucketize", bad)
    with pytest.raises(AssertionError):
        TL.test_bucketize_matches_stable_argsort_and_counts()


def test_wrong_nibble_order_is_caught(monkeypatch):
    monkeypatch.setattr(C, "pack_e2m1", lambda c: (np.asarray(c)[..., 1::2] & 0xF) | ((np.asarray(c)[..., 0::2] & 0xF) << 4))
    with pytest.raises(AssertionError):
        TC.test_fp4_pack_roundtrip_and_nibble_order()


def _combine_f64(o_bf16, slot_of):
    slot_of = np.asarray(slot_of)
    T, k = slot_of.shape
    acc = np.zeros((T, o_bf16.shape[1]), np.float64)
    for j in range(k):
        p = slot_of[:, j]
        acc[p >= 0] += C.bf16_value(o_bf16[p[p >= 0]])
    return C.bf16_bits(acc.astype(np.float32))


def _combine_reversed(o_bf16, slot_of):
    return _ORIG_COMBINE(o_bf16, np.asarray(slot_of)[:, ::-1])


_ORIG_COMBINE = M.combine


@pytest.mark.parametrize("patch", [_combine_f64, _combine_reversed], ids=["float64_sum", "reversed_slots"])
def test_combine_order_and_precision_mistakes_are_caught(monkeypatch, patch):
    monkeypatch.setattr(M, "combine", patch)
    with pytest.raises(AssertionError):
        TL.test_combine_adds_in_slot_order_in_fp32()


# ---------------------------------------------------------------- block-FP8 oracle

from oracle import blockfp8 as B  # noqa: E402
from tests import test_oracle_blockfp8 as TB  # noqa: E402

_ORIG_B_SCALE = B._scale
_ORIG_B_DQW = B.dequant_weights


def _scale_480(amax):
    s = (np.asarray(amax, np.float64) / 480.0).astype(np.float32)
    return np.where(np.asarray(amax) == 0, np.float32(1.0), s).astype(np.float32)


def _dq_weights_transposed_scales(codes, s):
    s = np.asarray(s)
    if s.shape[-1] == s.shape[-2]:
        s = np.swapaxes(s, -1, -2)
    return _ORIG_B_DQW(codes, s)


def test_block_scale_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(B, "_scale", _scale_480)
    with pytest.raises(AssertionError):
        TB.test_block_scale_is_amax_over_448_in_float32()


@pytest.mark.slow
@pytest.mark.parametrize("patch", ["transposed_block_scales", "dropped_topk_weight"])
def test_block_fp8_layer_mistakes_are_caught(monkeypatch, patch):
    if patch == "transposed_block_scales":
        # W2 of the tiny shape is one 128 x 128 block per expert, so transpose W13's
        # [2, 1] scale grid instead: swap which half of the gate/up rows each scale covers
        def dq(codes, s):
            s = np.asarray(s)
            if s.shape[-2] == 2:
                s = s[..., ::-1, :]
            return _ORIG_B_DQW(codes, s)
        monkeypatch.setattr(B, "dequant_weights", dq)
    else:
        monkeypatch.setattr(M, "silu_mul_weight", _dropped_weight)
    with pytest.raises(AssertionError):
        TB._compare_with_brute()
