"""An independent, loop-by-loop float64 model of the layer for tiny inputs.

It shares nothing with oracle/: E4M3 rounding comes from torch's float8_e4m3fn
cast, E2M1 rounding and the block exponent from exact rational search, dot
products from math.fsum (exact), BF16 rounding from torch's bfloat16 cast.
Only meant for shapes with a few thousand multiply-adds.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
             Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def f32(x: float) -> float:
    return float(np.float32(x))


def bf16_round(x: float) -> int:
    t = torch.tensor([x], dtype=torch.float32).to(torch.bfloat16)
    return int(t.view(torch.int16).item()) & 0xFFFF


def bf16_to_float(bits: int) -> float:
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def e4m3_round(x: float) -> int:
    return int(torch.tensor([x], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item())


def e4m3_to_float(code: int) -> float:
    return float(torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item())


def e2m1_round(x: Fraction, negative: bool) -> int:
    mag = abs(x)
    best, bestd = 0, None
    for c, m in enumerate(E2M1_MAGS):
        d = abs(mag - m)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (8 if negative else 0)


def e2m1_to_fraction(code: int) -> Fraction:
    v = E2M1_MAGS[code & 7]
    return -v if code & 8 else v


def min_exponent(amax: Fraction, q: Fraction) -> int:
    if amax == 0:
        return 0
    e = -160
    while amax > q * Fraction(2) ** e:
        e += 1
    return max(-127, min(127, e))


def quant_group(vals, fmt):
    """vals: list of 32 floats (exact) -> (codes, scale byte)."""
    fr = [Fraction(v) for v in vals]
    q = Fraction(448) if fmt == "e4m3" else Fraction(6)
    e = min_exponent(max(abs(v) for v in fr), q)
    s = Fraction(2) ** e
    codes = []
    for v, fv in zip(vals, fr):
        if fmt == "e4m3":
            codes.append(e4m3_round(math.ldexp(v, -e)))
        else:
            codes.append(e2m1_round(fv / s, math.copysign(1.0, v) < 0))
    return codes, e + 127


def dq_e4m3(code, sbyte):
    return e4m3_to_float(code) * 2.0 ** (sbyte - 127)


def dq_e2m1(code, sbyte):
    return float(e2m1_to_fraction(code)) * 2.0 ** (sbyte - 127)


def quant_matrix(rows, fmt):
    """rows: list of lists of floats -> (codes, scales) as nested lists."""
    codes, scales = [], []
    for r in rows:
        cr, sr = [], []
        for g in range(0, len(r), 32):
            c, s = quant_group(r[g:g + 32], fmt)
            cr += c
            sr.append(s)
        codes.append(cr)
        scales.append(sr)
    return codes, scales


def layer(x_bits, w13_bits, w2_bits, topk, I, logits=None, topk_idx=None,
          topk_w=None, score_fn=0, renorm=True):
    """Returns dict with idx, w, counts, xq, xsf, hq (per (t, j)), o (per (t, j)), y."""
    T, H = len(x_bits), len(x_bits[0])
    E = len(w13_bits)
    # routing
    if logits is not None:
        idx, wts = [], []
        for t in range(T):
            row = [float(v) for v in logits[t]]
            order = sorted(range(E), key=lambda e: (-row[e], e))[:topk]
            if score_fn == 0:
                m = max(row)
                z = [math.exp(v - m) for v in row]
                tot = math.fsum(z)
                s = [z[e] / tot for e in order]
            else:
                s = [1.0 / (1.0 + math.exp(-row[e])) for e in order]
            if renorm:
                tot = math.fsum(s)
                s = [v / tot for v in s]
            idx.append(order)
            wts.append([f32(v) for v in s])
    else:
        idx = [[int(v) for v in r] for r in topk_idx]
        wts = [[float(v) for v in r] for r in topk_w]
    counts = [0] * E
    for t in range(T):
        for j in range(topk):
            if idx[t][j] >= 0:
                counts[idx[t][j]] += 1
    # activation quantisation
    xf = [[bf16_to_float(int(b)) for b in row] for row in x_bits]
    xq, xsf = quant_matrix(xf, "e4m3")
    # weights
    wq13, ws13, wq2, ws2 = [], [], [], []
    for e in range(E):
        m13 = [[bf16_to_float(int(b)) for b in row] for row in w13_bits[e]]
        m2 = [[bf16_to_float(int(b)) for b in row] for row in w2_bits[e]]
        c, s = quant_matrix(m13, "e2m1")
        wq13.append(c); ws13.append(s)
        c, s = quant_matrix(m2, "e2m1")
        wq2.append(c); ws2.append(s)
    hq, hsf, o = {}, {}, {}
    y = []
    for t in range(T):
        a = [dq_e4m3(xq[t][h], xsf[t][h // 32]) for h in range(H)]
        acc_y = 0.0
        for j in range(topk):
            e = idx[t][j]
            if e < 0:
                continue
            acc1 = []
            for n in range(2 * I):
                b = [dq_e2m1(wq13[e][n][h], ws13[e][n][h // 32]) for h in range(H)]
                acc1.append(f32(math.fsum(a[h] * b[h] for h in range(H))))
            h_row = []
            for i in range(I):
                g, u = acc1[i], acc1[I + i]
                silu = g / (1.0 + math.exp(-g)) if g > -700 else 0.0 * g
                h_row.append(f32(silu * u * wts[t][j]))
            c, s = quant_matrix([h_row], "e4m3")
            hq[(t, j)], hsf[(t, j)] = c[0], s[0]
            a2 = [dq_e4m3(c[0][i], s[0][i // 32]) for i in range(I)]
            out = []
            for n in range(H):
                b = [dq_e2m1(wq2[e][n][i], ws2[e][n][i // 32]) for i in range(I)]
                out.append(bf16_round(f32(math.fsum(a2[i] * b[i] for i in range(I)))))
            o[(t, j)] = out
        row = []
        for n in range(H):
            acc = np.float32(0.0)
            for j in range(topk):
                if idx[t][j] >= 0:
                    acc = np.float32(acc + np.float32(bf16_to_float(o[(t, j)][n])))
            row.append(bf16_round(float(acc)))
        y.append(row)
    return dict(idx=idx, w=wts, counts=counts, xq=xq, xsf=xsf, hq=hq, hsf=hsf,
                o=o, y=y, wq13=wq13, ws13=ws13, wq2=wq2, ws2=ws2)


# ---------------------------------------------------------------- block-FP8 weights

def f32_of_fraction(x: Fraction) -> float:
    """x rounded to float32, nearest even, by exact search between float32 neighbours."""
    if x == 0:
        return 0.0
    a = float(np.float32(float(x)))            # within one float32 step of the answer
    cands = {a, float(np.nextafter(np.float32(a), np.float32(np.inf))),
             float(np.nextafter(np.float32(a), np.float32(-np.inf)))}
    best = min(cands, key=lambda c: (abs(Fraction(c) - x),
                                     int(np.array([c], np.float32).view(np.uint32)[0]) & 1))
    return best


def quant_fp8_block(vals):
    """vals: the exact values of one block -> (E4M3 codes, float32 scale): the scale is
    max|v| / 448 rounded to float32 (1 for an all-zero block), each code the E4M3 value
    nearest to v / s rounded to float32 (torch's cast), clamped to +-448."""
    amax = max(abs(Fraction(v)) for v in vals)
    s = f32_of_fraction(amax / 448) if amax else 1.0
    codes = []
    for v in vals:
        q = f32_of_fraction(Fraction(v) / Fraction(s))
        codes.append(e4m3_round(max(-448.0, min(448.0, q))))
    return codes, s


def layer_fp8b(x_bits, w13_bits, w2_bits, topk, I, logits):
    """Loop model of the block-FP8 variant (128 x 128 weight blocks, 1 x 128 activation
    groups, float32 scales), softmax routing renormalised.  Returns y and hq by (t, j)."""
    T, H = len(x_bits), len(x_bits[0])
    E = len(w13_bits)
    B = 128

    def qrow(row):
        codes, scales = [], []
        for g in range(0, len(row), B):
            c, s = quant_fp8_block(row[g:g + B])
            codes += c
            scales.append(s)
        return codes, scales

    def qmat(m):
        n, k = len(m), len(m[0])
        codes = [[0] * k for _ in range(n)]
        scales = [[0.0] * (k // B) for _ in range(n // B)]
        for bi in range(n // B):
            for bj in range(k // B):
                vals = [m[bi * B + r][bj * B + c] for r in range(B) for c in range(B)]
                cs, s = quant_fp8_block(vals)
                scales[bi][bj] = s
                for r in range(B):
                    for c in range(B):
                        codes[bi * B + r][bj * B + c] = cs[r * B + c]
        return codes, scales

    idx, wts = [], []
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:topk]
        m = max(row)
        z = [math.exp(v - m) for v in row]
        tot = math.fsum(z)
        s = [z[e] / tot for e in order]
        tot = math.fsum(s)
        idx.append(order)
        wts.append([f32(v / tot) for v in s])
    W13, W2 = [], []
    for e in range(E):
        W13.append(qmat([[bf16_to_float(int(b)) for b in r] for r in w13_bits[e]]))
        W2.append(qmat([[bf16_to_float(int(b)) for b in r] for r in w2_bits[e]]))
    hq, y = {}, []
    o = {}
    for t in range(T):
        xc, xs = qrow([bf16_to_float(int(b)) for b in x_bits[t]])
        # dequantised values and their products as exact rationals (a float32 scale
        # times a code has up to 28 significant bits, a product up to 56)
        a = [Fraction(e4m3_to_float(xc[h])) * Fraction(xs[h // B]) for h in range(H)]
        for j in range(topk):
            e = idx[t][j]
            (c13, s13), (c2, s2) = W13[e], W2[e]
            acc1 = [f32_of_fraction(sum(a[h] * Fraction(e4m3_to_float(c13[n][h])) * Fraction(s13[n // B][h // B])
                                        for h in range(H)))
                    for n in range(2 * I)]
            h_row = []
            for i in range(I):
                g, u = acc1[i], acc1[I + i]
                silu = g / (1.0 + math.exp(-g)) if g > -700 else 0.0 * g
                h_row.append(f32(silu * u * wts[t][j]))
            hc, hs = qrow(h_row)
            hq[(t, j)] = (hc, hs)
            a2 = [Fraction(e4m3_to_float(hc[i])) * Fraction(hs[i // B]) for i in range(I)]
            o[(t, j)] = [bf16_round(f32_of_fraction(sum(a2[i] * Fraction(e4m3_to_float(c2[n][i])) *
                                                        Fraction(s2[n // B][i // B]) for i in range(I))))
                         for n in range(H)]
        row = []
        for n in range(H):
            acc = np.float32(0.0)
            for j in range(topk):
                acc = np.float32(acc + np.float32(bf16_to_float(o[(t, j)][n])))
            row.append(bf16_round(float(acc)))
        y.append(row)
    return dict(idx=idx, w=wts, hq=hq, y=y)
