"""Pins for oracle/moe_ref.py against brute force, library routines and invariants."""
import math

import numpy as np
import pytest

import moe_workloads as W
from oracle import codecs as C
from oracle import moe_ref as M
from tests import brute_force as BF


def _quantised_weights(w: W.Workload):
    w13, w2 = W.gen_weights(w, threads=4)
    w13q, w13sf = M.pack_weights(w13)
    w2q, w2sf = M.pack_weights(w2)
    return w13, w2, w13q, w13sf, w2q, w2sf


# ------------------------------------------------------------ routing

@pytest.mark.parametrize("score_fn", [M.SOFTMAX, M.SIGMOID])
@pytest.mark.parametrize("renorm", [True, False])
def test_route_matches_sort_based_brute_force(score_fn, renorm):
    rng = np.random.default_rng(0)
    T, E, k = 37, 11, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[3, :] = 0.5                      # all tied: lowest indices win, in order
    logits[4, 2] = logits[4, 7] = 9.0       # two-way tie at the top
    idx, w = M.route(logits, k, score_fn, renorm)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        assert idx[t].tolist() == order
        l = logits[t].astype(np.float64)
        if score_fn == M.SOFTMAX:
            p = [math.exp(v) / math.fsum(math.exp(u) for u in l) for v in l]
        else:
            p = [1 / (1 + math.exp(-v)) for v in l]
        s = [p[e] for e in order]
        if renorm:
            s = [v / math.fsum(s) for v in s]
        np.testing.assert_allclose(w[t], np.float32(s), rtol=2e-7, atol=0)
    assert idx[3].tolist() == [0, 1, 2]
    assert idx[4].tolist()[:2] == [2, 7]


def test_route_weights_sum_to_one_and_ids_distinct():
    w = W.WORKLOADS["decode"]
    idx, wt = M.route(W.gen_logits(w), w.topk, M.SOFTMAX, True)
    assert np.allclose(wt.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert all(len(set(r)) == w.topk for r in idx.tolist())


def test_route_softmax_renorm_equals_softmax_over_chosen():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((50, 32)).astype(np.float32)
    idx, wt = M.route(logits, 8, M.SOFTMAX, True)
    chosen = np.take_along_axis(logits.astype(np.float64), idx, 1)
    z = np.exp(chosen - chosen.max(1, keepdims=True))
    np.testing.assert_allclose(wt, (z / z.sum(1, keepdims=True)).astype(np.float32), rtol=3e-7)


def test_route_topk_equals_E_selects_everything():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((9, 6)).astype(np.float32)
    idx, wt = M.route(logits, 6, M.SIGMOID, True)
    assert all(sorted(r) == list(range(6)) for r in idx.tolist())


# ------------------------------------------------------------ bucketize

def test_bucketize_matches_stable_argsort_and_counts():
    w = W.WORKLOADS["dsv3_skewed"].with_tokens(512)
    idx, _ = M.route(W.gen_logits(w), w.topk)
    counts, offsets, slot_src, slot_of = M.bucketize(idx, w.E)
    flat = idx.reshape(-1)
    assert counts.sum() == w.T * w.topk                     # counts sum to T*k
    assert np.array_equal(counts, np.bincount(flat, minlength=w.E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=w.E))]))
    assert np.array_equal(slot_src, np.argsort(flat, kind="stable"))   # library stable sort
    assert np.array_equal(slot_src[slot_of.reshape(-1)], np.arange(flat.size))


def test_bucketize_skips_masked_and_handles_empty_experts():
    idx = np.array([[2, -1], [2, 0], [-1, -1], [0, 2]], np.int32)
    counts, offsets, slot_src, slot_of = M.bucketize(idx, 4)
    assert counts.tolist() == [2, 0, 3, 0]
    assert offsets.tolist() == [0, 2, 2, 5, 5]
    assert slot_src.tolist() == [3, 6, 0, 2, 7]
    assert slot_of.tolist() == [[2, -1], [3, 0], [-1, -1], [1, 4]]


# ------------------------------------------------------------ quantisation steps

def test_quant_act_matches_brute_force():
    w = W.WORKLOADS["tiny"]
    x = W.gen_x(w)[:4]
    xq, xsf = M.quant_act(x)
    bq, bs = BF.quant_matrix([[BF.bf16_to_float(int(b)) for b in r] for r in x], "e4m3")
    assert np.array_equal(xq, np.array(bq, np.uint8))
    assert np.array_equal(xsf, np.array(bs, np.uint8))


def test_pack_weights_matches_brute_force():
    w = W.Workload("p", T=1, H=64, I=32, E=1, topk=1)
    w13 = W.gen_expert_w13(w, 0)[:6]
    q, s = M.pack_weights(w13)
    bq, bs = BF.quant_matrix([[BF.bf16_to_float(int(b)) for b in r] for r in w13], "e2m1")
    assert np.array_equal(C.unpack_e2m1(q), np.array(bq, np.uint8))
    assert np.array_equal(s, np.array(bs, np.uint8))


# ------------------------------------------------------------ whole layer vs brute force

def _compare_with_brute(w: W.Workload, external=False, score_fn=M.SOFTMAX, mask=0.0):
    w13, w2, w13q, w13sf, w2q, w2sf = _quantised_weights(w)
    x = W.gen_x(w)
    if external:
        idx, wt = W.gen_external_topk(w, mask)
        out = M.forward(x, w13q, w13sf, w2q, w2sf, topk=w.topk, I=w.I, topk_idx=idx, topk_w=wt)
        bf = BF.layer(x, w13, w2, w.topk, w.I, topk_idx=idx, topk_w=wt)
    else:
        logits = W.gen_logits(w)
        out = M.forward(x, w13q, w13sf, w2q, w2sf, topk=w.topk, I=w.I, logits=logits,
                        score_fn=score_fn)
        bf = BF.layer(x, w13, w2, w.topk, w.I, logits=logits, score_fn=score_fn)
    # the brute force re-derives weight codes independently
    for e in range(w.E):
        assert np.array_equal(C.unpack_e2m1(w13q[e]), np.array(bf["wq13"][e], np.uint8))
        assert np.array_equal(w13sf[e], np.array(bf["ws13"][e], np.uint8))
        assert np.array_equal(C.unpack_e2m1(w2q[e]), np.array(bf["wq2"][e], np.uint8))
    assert out["topk_idx"].tolist() == bf["idx"]
    np.testing.assert_allclose(out["topk_w"], np.array(bf["w"], np.float32), rtol=2e-7)
    assert out["counts"].tolist() == bf["counts"]
    assert np.array_equal(out["xq"], np.array(bf["xq"], np.uint8))
    assert np.array_equal(out["xsf"], np.array(bf["xsf"], np.uint8))
    for (t, j), hq in bf["hq"].items():
        p = out["slot_of"][t, j]
        assert np.array_equal(out["hq"][p], np.array(hq, np.uint8)), (t, j)
        assert np.array_equal(out["hsf"][p], np.array(bf["hsf"][(t, j)], np.uint8))
        assert np.array_equal(out["o"][p], np.array(bf["o"][(t, j)], np.uint16))
    assert np.array_equal(out["y"], np.array(bf["y"], np.uint16))


@pytest.mark.parametrize("w", W.tiny_shapes()[::5], ids=lambda w: w.name)
def test_forward_matches_brute_force_tiny_shapes(w):
    _compare_with_brute(w)


def test_forward_matches_brute_force_sigmoid():
    _compare_with_brute(W.Workload("s", T=5, H=64, I=32, E=4, topk=2, score_fn=M.SIGMOID),
                        score_fn=M.SIGMOID)


def test_forward_matches_brute_force_external_masked_topk():
    _compare_with_brute(W.Workload("m", T=9, H=32, I=32, E=3, topk=2), external=True, mask=0.3)


@pytest.mark.slow
def test_forward_matches_brute_force_tiny_workload_sample():
    # the tiny workload itself, restricted to its first 4 tokens
    w = W.WORKLOADS["tiny"].with_tokens(4)
    _compare_with_brute(w)


# ------------------------------------------------------------ invariants

def test_gemm1_accumulator_is_rounded_exact_sum():
    w = W.Workload("g", T=3, H=96, I=32, E=1, topk=1)
    _, _, w13q, w13sf, _, _ = _quantised_weights(w)
    x = W.gen_x(w)
    xq, xsf = M.quant_act(x)
    _, _, acc1, _ = M.expert_rows(xq, xsf, np.ones(3, np.float32), w13q[0], w13sf[0],
                                  np.zeros((w.H, w.I // 2), np.uint8),
                                  np.full((w.H, w.I // 32), 127, np.uint8), w.I)
    codes = C.unpack_e2m1(w13q[0])
    for r in range(3):
        a = [BF.dq_e4m3(int(xq[r, h]), int(xsf[r, h // 32])) for h in range(w.H)]
        for n in range(2 * w.I):
            b = [BF.dq_e2m1(int(codes[n, h]), int(w13sf[0][n, h // 32])) for h in range(w.H)]
            assert acc1[r, n] == np.float32(math.fsum(x * y for x, y in zip(a, b)))


def test_top1_unit_weight_is_single_expert_mlp():
    """k = 1, w = 1: every token's y is the quantised dense MLP of its expert."""
    w = W.Workload("mlp", T=6, H=64, I=64, E=3, topk=1)
    w13, w2, w13q, w13sf, w2q, w2sf = _quantised_weights(w)
    x = W.gen_x(w)
    idx = np.array([[0], [2], [1], [2], [0], [0]], np.int32)
    out = M.forward(x, w13q, w13sf, w2q, w2sf, topk=1, I=w.I, topk_idx=idx,
                    topk_w=np.ones((6, 1), np.float32))
    for t in range(w.T):
        e = idx[t, 0]
        xq, xsf = BF.quant_matrix([[BF.bf16_to_float(int(b)) for b in x[t]]], "e4m3")
        a = [BF.dq_e4m3(xq[0][h], xsf[0][h // 32]) for h in range(w.H)]
        b13 = C.dequantize_blocks(C.unpack_e2m1(w13q[e]), w13sf[e], "e2m1")
        acc = [np.float32(math.fsum(a[h] * b13[n, h] for h in range(w.H))) for n in range(2 * w.I)]
        h = [np.float32(float(acc[i]) / (1 + math.exp(-float(acc[i]))) * float(acc[w.I + i]))
             for i in range(w.I)]
        hq, hs = BF.quant_matrix([[float(v) for v in h]], "e4m3")
        a2 = [BF.dq_e4m3(hq[0][i], hs[0][i // 32]) for i in range(w.I)]
        b2 = C.dequantize_blocks(C.unpack_e2m1(w2q[e]), w2sf[e], "e2m1")
        y = [BF.bf16_round(float(np.float32(math.fsum(a2[i] * b2[n, i] for i in range(w.I)))))
             for n in range(w.H)]
        assert out["y"][t].tolist() == y


def test_token_permutation_permutes_y_exactly():
    w = W.WORKLOADS["tiny"]
    _, _, w13q, w13sf, w2q, w2sf = _quantised_weights(w)
    x, logits = W.gen_x(w), W.gen_logits(w)
    perm = np.random.default_rng(3).permutation(w.T)
    a = M.forward(x, w13q, w13sf, w2q, w2sf, topk=w.topk, I=w.I, logits=logits)
    b = M.forward(x[perm], w13q, w13sf, w2q, w2sf, topk=w.topk, I=w.I, logits=logits[perm])
    assert np.array_equal(a["y"][perm], b["y"])


def test_token_subset_matches_full_forward():
    w = W.WORKLOADS["tiny"]
    _, _, w13q, w13sf, w2q, w2sf = _quantised_weights(w)
    x, logits = W.gen_x(w), W.gen_logits(w)
    full = M.forward(x, w13q, w13sf, w2q, w2sf, topk=w.topk, I=w.I, logits=logits)
    toks = [0, 5, 63]
    sub = M.forward(x, w13q, w13sf, w2q, w2sf, topk=w.topk, I=w.I, logits=logits, tokens=toks)
    assert np.array_equal(full["y"][toks], sub["y"][toks])


def test_combine_adds_in_slot_order_in_fp32():
    """y[t] = BF16 of the float32 sum of the token's rows in slot order j = 0..k-1
    ([MegaMoE notes] "L2 epilogue"; the q6 reading).  With rows 1, 2^-8, 2^-24,
    2^-24 (all BF16), the float32 sum in slot order stays at 1 + 2^-8: each
    2^-24 is half a float32 ulp there and rounds back to the even neighbour.  That
    is the midpoint of BF16 1 and 1 + 2^-7, which rounds to the even 1.0.  Adding
    the same rows in reverse order (2^-24 + 2^-24 = 2^-23 first) or exactly gives
    1 + 2^-8 + 2^-23, above the midpoint: BF16 1 + 2^-7."""
    vals = np.array([[1.0], [2.0 ** -8], [2.0 ** -24], [2.0 ** -24]], np.float32)
    o = C.bf16_bits(vals)
    assert np.array_equal(C.bf16_value(o), vals)             # the rows are BF16 values
    y = M.combine(o, np.array([[0, 1, 2, 3]]))
    assert C.bf16_value(y)[0, 0] == 1.0
    y_rev = M.combine(o, np.array([[3, 2, 1, 0]]))             # the same rows, slots reversed
    assert C.bf16_value(y_rev)[0, 0] == 1.0 + 2.0 ** -7


def test_interleave_w13_matches_the_pages_layout():
    """[MegaMoE notes] "原始权重布局": after the gran = 8 interleave the N dimension
    reads gate0 (8 rows), up0 (8), gate1 (8), up1 (8), ...; every 8 gate rows are
    followed by the 8 up rows of the same columns."""
    I = 32
    rows = np.arange(2 * I, dtype=np.int64)
    q = np.repeat(rows[None, :, None], 3, axis=2)           # [1, 2I, 3], row r holds r
    sf = np.repeat(rows[None, :, None], 2, axis=2)
    iq, isf = M.interleave_w13(q, sf)
    expect = np.concatenate([np.r_[8 * i:8 * i + 8, I + 8 * i:I + 8 * i + 8] for i in range(I // 8)])
    assert np.array_equal(iq[0, :, 0], expect)
    assert np.array_equal(isf[0, :, 1], expect)
    assert list(expect[:32]) == list(range(0, 8)) + list(range(32, 40)) + list(range(8, 16)) + list(range(40, 48))
    assert np.array_equal(np.sort(expect), rows)             # a permutation of the rows
