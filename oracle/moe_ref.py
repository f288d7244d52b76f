"""Plain CPU reference of the fused FP8 x FP4 top-k MoE layer.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The layer, as the pages describe it ([MegaMoE notes] "Dispatch阶段" flow chart
and "GEMM"/"Activate"/"Combine"; [MonoMoe] §1 phases 1-5):

  1. route        per token: scores over E experts (softmax or sigmoid), pick the
                  k largest, optionally renormalise the k weights  ([MonoMoe] §1
                  phase 1)
  2. bucketize    counting sort of the T*k (token, slot) pairs by expert: counts,
                  exclusive prefix sum, scatter of t*k + j into per-expert
                  contiguous slots ([Counting sort] 2.1-2.3; entries < 0 are
                  skipped, 7.1)
  3. quant_act    x BF16 -> FP8 E4M3 codes + one UE8M0 scale per 32 hidden
                  ([MegaMoE notes] "Dispatch阶段")
  4. GEMM1        per expert, slot rows x W13^T with W13 = [gate; up] FP4 E2M1 +
                  UE8M0 per 32 along K, FP32 accumulation ([MegaMoE notes] "GEMM",
                  flow chart; [MegaMoE fusion] "L1/L2 交错" table)
  5. epilogue     h = silu(gate) * up * topk_weight on the FP32 accumulators,
                  re-quantised to FP8 + UE8M0 per 32 along I ([MegaMoE notes]
                  flow chart; [Warp spec] L1 epilogue excerpt)
  6. GEMM2        per expert, h rows x W2^T (FP4), FP32 accumulation, rounded to
                  BF16 ([MegaMoE notes] "L2 epilogue")
  7. combine      y[t] = BF16(sum over the token's k rows, FP32, slot order)
                  ([MegaMoE notes] "L2 epilogue"; [Warp spec] combine excerpt)

Precision: accumulations are formed in float64 (exact for these operands) and
rounded once to float32, the accumulator precision the pages give; the
epilogue is evaluated in float64 on those float32 values and rounded once to
float32, the precision the FP8 decision is taken in; BF16 results are rounded
from float32 (nearest even).  The combine adds float32 values in slot order in
float32, as the pages do.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import codecs as C

SOFTMAX = 0
SIGMOID = 1


# ------------------------------------------------------------------ 1. route

def route(logits, topk: int, score_fn: int = SOFTMAX, renorm: bool = True):
    """Top-k routing.

    Selection compares the float32 logits themselves: softmax and sigmoid are
    both increasing, so the k largest scores are the k largest logits.  Slots
    are ordered by decreasing logit, equal logits by increasing expert index.

    Weights (float64, rounded once to float32):
      softmax: p = softmax over all E; renorm: p_j / sum over the chosen p
      sigmoid: s = 1/(1+exp(-l));      renorm: s_j / sum over the chosen s
    Returns (topk_idx int32 [T, k], topk_w float32 [T, k]).
    """
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    assert 1 <= topk <= E
    l = l32.astype(np.float64)
    order = np.argsort(-l, axis=1, kind="stable")        # stable: ties -> lower index
    idx = order[:, :topk]
    chosen = np.take_along_axis(l, idx, axis=1)
    if score_fn == SOFTMAX:
        z = np.exp(l - l.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        s = np.take_along_axis(p, idx, axis=1)
    elif score_fn == SIGMOID:
        s = 1.0 / (1.0 + np.exp(-chosen))
    else:
        raise ValueError("score_fn")
    if renorm:
        s = s / s.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), s.astype(np.float32)


# ------------------------------------------------------------------ 2. bucketize

def bucketize(topk_idx, E: int):
    """Counting sort of (token, slot) pairs by expert.

    Pair (t, j) has flat id f = t*k + j and expert e = topk_idx[t, j]; pairs with
    e < 0 are skipped.  Returns
      counts   int32 [E]     pairs per expert
      offsets  int32 [E+1]   exclusive prefix sum of counts
      slot_src int32 [N]     f of each pair, expert segments in expert order,
                             ascending f inside a segment (N = valid pairs)
      slot_of  int32 [T, k]  position of pair (t, j) in slot_src, -1 if skipped
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(E, np.int64)
    for f in range(flat.size):                     # count
        e = flat[f]
        if e >= 0:
            assert e < E
            counts[e] += 1
    offsets = np.zeros(E + 1, np.int64)            # exclusive prefix sum
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()                    # scatter
    slot_src = np.zeros(offsets[E], np.int64)
    slot_of = np.full(T * k, -1, np.int64)
    for f in range(flat.size):
        e = flat[f]
        if e >= 0:
            slot_src[cursor[e]] = f
            slot_of[f] = cursor[e]
            cursor[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            slot_src.astype(np.int32), slot_of.reshape(T, k).astype(np.int32))


# ------------------------------------------------------------------ 3. quantisation

def quant_act(x_bf16_bits):
    """BF16 rows [T, H] -> (E4M3 codes uint8 [T, H], UE8M0 uint8 [T, H/32])."""
    v = C.bf16_value(x_bf16_bits).astype(np.float64)
    return C.quantize_blocks(v, "e4m3")


def pack_weights(w_bf16_bits):
    """BF16 weights [..., N, K] -> (packed E2M1 uint8 [..., N, K/2], UE8M0 [..., N, K/32]).

    One scale per 32 consecutive K elements of a row; rows are not grouped
    ([MegaMoE notes] "Expert矩阵权重量化").  Element 2i sits in the low nibble.
    """
    v = C.bf16_value(w_bf16_bits).astype(np.float64)
    codes, sf = C.quantize_blocks(v, "e2m1")
    return C.pack_e2m1(codes), sf


def interleave_w13(w13q, w13sf, gran: int = 8):
    """The pages' offline gate/up row interleave of W13 ([MegaMoE notes]
    "原始权重布局", "_interleave_l1_weights" with gran = 8): the canonical rows are
    gate [0, I) then up [I, 2I); the interleaved rows alternate blocks of ``gran``
    gate rows and the ``gran`` up rows of the same columns, so rows
    [2 gran i, 2 gran i + gran) are gate rows [gran i, gran i + gran) and rows
    [2 gran i + gran, 2 gran (i + 1)) are up rows [gran i, gran i + gran).
    Works on codes [..., 2I, H/2] and per-row scales [..., 2I, H/32] alike."""
    out = []
    for a in (np.asarray(w13q), np.asarray(w13sf)):
        two_i = a.shape[-2]
        I = two_i // 2
        assert two_i % 2 == 0 and I % gran == 0
        b = np.empty_like(a)
        for i in range(I // gran):
            g0 = gran * i
            b[..., 2 * g0:2 * g0 + gran, :] = a[..., g0:g0 + gran, :]
            b[..., 2 * g0 + gran:2 * g0 + 2 * gran, :] = a[..., I + g0:I + g0 + gran, :]
        out.append(b)
    return out[0], out[1]


def dequant_weights(packed, sf) -> np.ndarray:
    return C.dequantize_blocks(C.unpack_e2m1(packed), sf, "e2m1")


# ------------------------------------------------------------------ 4-7. expert MLP

def silu_mul_weight(g32, u32, w32) -> np.ndarray:
    """h = silu(g) * u * w, silu(g) = g / (1 + exp(-g)); float64, rounded to float32."""
    g = np.asarray(g32, dtype=np.float64)
    u = np.asarray(u32, dtype=np.float64)
    w = np.asarray(w32, dtype=np.float64)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return (silu * u * w).astype(np.float32)


def expert_rows(xq_rows, xsf_rows, wts, w13q, w13sf, w2q, w2sf, I: int):
    """GEMM1 -> epilogue -> GEMM2 for rows that all go to one expert.

    xq_rows/xsf_rows: the rows' activation codes and scales; wts: their top-k
    weights (float32).  Returns (hq uint8 [n, I], hsf uint8 [n, I/32], acc1
    float32 [n, 2I], out_bf16 uint16 [n, H]).
    """
    a = C.dequantize_blocks(xq_rows, xsf_rows, "e4m3")          # [n, H] exact
    b13 = dequant_weights(w13q, w13sf)                           # [2I, H] exact
    acc1 = (a @ b13.T).astype(np.float32)                        # FP32 accumulator
    h = silu_mul_weight(acc1[:, :I], acc1[:, I:], np.asarray(wts, np.float32)[:, None])
    hq, hsf = C.quantize_blocks(h.astype(np.float64), "e4m3")
    a2 = C.dequantize_blocks(hq, hsf, "e4m3")                   # [n, I]
    b2 = dequant_weights(w2q, w2sf)                              # [H, I]
    acc2 = (a2 @ b2.T).astype(np.float32)
    return hq, hsf, acc1, C.bf16_bits(acc2)


def combine(o_bf16, slot_of) -> np.ndarray:
    """y[t] = BF16(sum_j o[slot_of[t, j]]) with float32 adds in slot order j = 0..k-1."""
    slot_of = np.asarray(slot_of)
    T, k = slot_of.shape
    H = o_bf16.shape[1]
    acc = np.zeros((T, H), np.float32)
    for j in range(k):
        p = slot_of[:, j]
        valid = p >= 0
        rows = np.zeros((T, H), np.float32)
        rows[valid] = C.bf16_value(o_bf16[p[valid]])
        acc = (acc + rows).astype(np.float32)
    return C.bf16_bits(acc)


def forward(x_bf16_bits, w13q, w13sf, w2q, w2sf, *, topk, I, logits=None,
            topk_idx=None, topk_w=None, score_fn=SOFTMAX, renorm=True, tokens=None,
            workers=None):
    """Whole layer.  Either ``logits`` [T, E] or ``topk_idx``/``topk_w`` [T, k].

    Weights are already quantised: w13q [E, 2I, H/2], w13sf [E, 2I, H/32],
    w2q [E, H, I/2], w2sf [E, H, I/32] (indexable by expert; a dict works).
    ``tokens`` restricts GEMMs and combine to those tokens (routing and
    bucketisation still cover all tokens); y rows of other tokens are zero.
    ``workers`` > 1 runs the per-expert steps on that many threads (each expert
    writes its own rows; the arithmetic is the same).
    Returns a dict of every intermediate.
    """
    x = np.asarray(x_bf16_bits, dtype=np.uint16)
    T, H = x.shape
    if logits is not None:
        E = np.asarray(logits).shape[1]
        topk_idx, topk_w = route(logits, topk, score_fn, renorm)
    else:
        E = len(w13q)
        topk_idx = np.asarray(topk_idx, np.int32)
        topk_w = np.asarray(topk_w, np.float32)
    counts, offsets, slot_src, slot_of = bucketize(topk_idx, E)
    xq, xsf = quant_act(x)

    N = int(offsets[E])
    want = np.ones(N, bool)
    if tokens is not None:
        sel = np.zeros(T, bool)
        sel[np.asarray(tokens)] = True
        want = sel[slot_src // topk]
    hq = np.zeros((N, I), np.uint8)
    hsf = np.zeros((N, I // 32), np.uint8)
    o = np.zeros((N, H), np.uint16)
    def one_expert(e):
        pos = np.arange(offsets[e], offsets[e + 1])
        pos = pos[want[pos]]
        if pos.size == 0:
            return
        f = slot_src[pos]
        t, j = f // topk, f % topk
        hq[pos], hsf[pos], _, o[pos] = expert_rows(
            xq[t], xsf[t], topk_w[t, j], w13q[e], w13sf[e], w2q[e], w2sf[e], I)

    if workers and workers > 1:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, range(E)))
    else:
        for e in range(E):
            one_expert(e)
    so = slot_of.copy()
    if tokens is not None:
        so[~sel] = -1
    y = combine(o, so)
    return dict(topk_idx=topk_idx, topk_w=topk_w, counts=counts, offsets=offsets,
                slot_src=slot_src, slot_of=slot_of, xq=xq, xsf=xsf, hq=hq, hsf=hsf,
                o=o, y=y)
