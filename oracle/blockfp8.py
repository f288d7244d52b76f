"""Plain CPU reference of the block-FP8 (128 x 128) weight variant of the layer.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[MonoMoe] (the fixed-shape paragraph and §1): the decode-shape kernel takes
block-FP8 weights with 128 x 128 blocks (E = 256, K = 2048, N = 512, at most 8
tokens); phase 2 quantises the BF16 input to FP8 with an activation scale;
phase 3 is the up-projection with SiLU, written back as FP8; phase 4 the
down-projection with FP32 partial sums; phase 5 the cast to BF16.  Routing,
bucketisation and the combine are those of the main path (moe_ref).

The page names the format only.  Readings (the plainest ones the rest supports):
  b1  weights: E4M3 codes [..., N, K]; one float32 scale per 128 x 128 block
      (128 rows x 128 K), [..., N/128, K/128]; value = code * scale.
  b2  activations (x, and h between the GEMMs): E4M3 codes, one float32 scale
      per row per 128 consecutive K elements, [..., rows, K/128].
  b3  the scale of a block is its largest magnitude divided by 448 (the largest
      finite E4M3 value), rounded to float32, so the largest element maps to
      +-448; an all-zero block gets scale 1.  Codes are E4M3 nearest-even of
      v / s rounded to float32 first (the float32 quotient a quantiser forms).
  b4  GEMMs: FP32 accumulation of the products of dequantised values.  Here
      they are formed in float64 and rounded once to float32; a dequantised
      value has up to 28 significant bits, so the float64 products and sums
      are within about 2^-45 of the exact sum of |products|, far below the
      float32 rounding the result is compared at.
  b5  the top-k weight is applied in the GEMM1 epilogue, h = silu(g) * u * w
      (as on the main path); the combine is the deterministic slot-order gather.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import codecs as C
from . import moe_ref as M

BLOCK = 128
E4M3_MAX = 448.0


def _scale(amax: np.ndarray) -> np.ndarray:
    """float32 scale of blocks with largest magnitude amax (b3): amax / 448 rounded
    to float32 (amax is a float32 value, so the float64 quotient rounded once is the
    correctly rounded float32 quotient); 1 for an all-zero block."""
    s = (np.asarray(amax, np.float64) / E4M3_MAX).astype(np.float32)
    return np.where(np.asarray(amax) == 0, np.float32(1.0), s).astype(np.float32)


def _codes(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E4M3 codes of v / s (b3): the quotient of two float32 values rounded to float32,
    then nearest-even onto the E4M3 grid (magnitudes above 448 clamp)."""
    q = (np.asarray(v, np.float64) / np.asarray(s, np.float64)).astype(np.float32)
    return C.e4m3_encode(q.astype(np.float64))


def quant_weights(w_bf16_bits):
    """BF16 weights [..., N, K] (N, K multiples of 128) -> (E4M3 codes uint8 [..., N, K],
    float32 scales [..., N/128, K/128]) (b1, b3)."""
    v = C.bf16_value(w_bf16_bits).astype(np.float32)
    *lead, N, K = v.shape
    assert N % BLOCK == 0 and K % BLOCK == 0
    blocks = v.reshape(*lead, N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=(-3, -1))
    s = _scale(amax)
    codes = _codes(blocks, s[..., :, None, :, None])
    return codes.reshape(v.shape), s


def quant_rows(v_f32):
    """float32 rows [..., K] (K a multiple of 128) -> (E4M3 codes uint8 [..., K], float32
    scales [..., K/128]), one scale per row per 128 elements (b2, b3)."""
    v = np.asarray(v_f32, np.float32)
    K = v.shape[-1]
    assert K % BLOCK == 0
    g = v.reshape(*v.shape[:-1], K // BLOCK, BLOCK)
    s = _scale(np.abs(g).max(axis=-1))
    return _codes(g, s[..., None]).reshape(v.shape), s


def quant_act(x_bf16_bits):
    """BF16 activations [T, H] -> (codes [T, H], float32 scales [T, H/128])."""
    return quant_rows(C.bf16_value(x_bf16_bits).astype(np.float32))


def dequant_weights(codes, s) -> np.ndarray:
    """code * scale of its 128 x 128 block, float64 [..., N, K] (exact)."""
    vals = C.E4M3_TABLE[np.asarray(codes).astype(np.int64)]
    *lead, N, K = vals.shape
    b = vals.reshape(*lead, N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    return (b * np.asarray(s, np.float64)[..., :, None, :, None]).reshape(vals.shape)


def dequant_rows(codes, s) -> np.ndarray:
    """code * scale of its row's 128-element group, float64 [..., K] (exact)."""
    vals = C.E4M3_TABLE[np.asarray(codes).astype(np.int64)]
    K = vals.shape[-1]
    g = vals.reshape(*vals.shape[:-1], K // BLOCK, BLOCK)
    return (g * np.asarray(s, np.float64)[..., None]).reshape(vals.shape)


def expert_rows(xq_rows, xsf_rows, wts, w13q, w13sf, w2q, w2sf, I: int):
    """GEMM1 -> epilogue -> GEMM2 for rows of one expert (b4, b5).  Returns (hq uint8
    [n, I], hsf float32 [n, I/128], acc1 float32 [n, 2I], out BF16 bits [n, H])."""
    a = dequant_rows(xq_rows, xsf_rows)                           # [n, H] exact
    b13 = dequant_weights(w13q, w13sf)                            # [2I, H] exact
    acc1 = (a @ b13.T).astype(np.float32)
    h = M.silu_mul_weight(acc1[:, :I], acc1[:, I:], np.asarray(wts, np.float32)[:, None])
    hq, hsf = quant_rows(h)
    a2 = dequant_rows(hq, hsf)
    b2 = dequant_weights(w2q, w2sf)                               # [H, I]
    acc2 = (a2 @ b2.T).astype(np.float32)
    return hq, hsf, acc1, C.bf16_bits(acc2)


def forward(x_bf16_bits, w13q, w13sf, w2q, w2sf, *, topk, I, logits=None, topk_idx=None,
            topk_w=None, score_fn=M.SOFTMAX, renorm=True, workers=None):
    """Whole layer with block-FP8 weights: w13q [E, 2I, H] codes, w13sf [E, 2I/128, H/128],
    w2q [E, H, I], w2sf [E, H/128, I/128] (indexable by expert).  Routing, the counting
    sort and the combine are moe_ref's.  Returns a dict of every intermediate."""
    x = np.asarray(x_bf16_bits, dtype=np.uint16)
    T, H = x.shape
    if logits is not None:
        E = np.asarray(logits).shape[1]
        topk_idx, topk_w = M.route(logits, topk, score_fn, renorm)
    else:
        E = len(w13q)
        topk_idx = np.asarray(topk_idx, np.int32)
        topk_w = np.asarray(topk_w, np.float32)
    counts, offsets, slot_src, slot_of = M.bucketize(topk_idx, E)
    xq, xsf = quant_act(x)
    N = int(offsets[E])
    hq = np.zeros((N, I), np.uint8)
    hsf = np.zeros((N, I // BLOCK), np.float32)
    o = np.zeros((N, H), np.uint16)

    def one_expert(e):
        pos = np.arange(offsets[e], offsets[e + 1])
        if pos.size == 0:
            return
        f = slot_src[pos]
        t, j = f // topk, f % topk
        hq[pos], hsf[pos], _, o[pos] = expert_rows(xq[t], xsf[t], topk_w[t, j], w13q[e], w13sf[e],
                                                   w2q[e], w2sf[e], I)

    if workers and workers > 1:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, range(E)))
    else:
        for e in range(E):
            one_expert(e)
    y = M.combine(o, slot_of)
    return dict(topk_idx=topk_idx, topk_w=topk_w, counts=counts, offsets=offsets, slot_src=slot_src,
                slot_of=slot_of, xq=xq, xsf=xsf, hq=hq, hsf=hsf, o=o, y=y)
