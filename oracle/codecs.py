"""Number formats used by the layer, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name the formats without defining them: activations are FP8 E4M3,
weights FP4 E2M1, and every group of 32 elements along K shares one UE8M0
(power-of-two) scale ([MegaMoE notes] "Dispatch阶段", "Expert矩阵权重量化";
[Warp spec] L1 epilogue excerpt).  They are read here as the OCP Microscaling
v1.0 formats:

  E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
               S.1111.111 is NaN; largest finite 448; subnormals m * 2^-9.
  E2M1:        1 sign, 2 exponent (bias 1), 1 mantissa bit;
               magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
  E8M0:        unsigned 8-bit exponent, value 2^(b - 127); b = 255 is NaN.

Block quantiser (the pages do not state how the scale is chosen from the
group's values; this is the reading used throughout): for a group v[0..31] and
a format whose largest finite magnitude is Q, the scale is the smallest power
of two s = 2^e with max|v| <= Q * s (e = 0 when the group is all zero), and each
element is v / s rounded to the nearest representable value, ties to the even
code, keeping the sign.  Exponents are clamped to the E8M0 range [-127, 127].

All arithmetic is float64 on values that are exact in float64, so every
rounding decision here is exact.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
GROUP = 32


# ---------------------------------------------------------------- decoding

def e4m3_value(code: int) -> float:
    """Value of one E4M3 code from the bit-field definition (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return s * (man / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e2m1_value(code: int) -> float:
    """Value of one E2M1 code (4 bits) from the bit-field definition."""
    s = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        return s * (man / 2.0) * 2.0 ** (1 - 1)
    return s * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(b):
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, b - 127).astype(np.float64)
    return np.where(b == 255, np.nan, out)


# ---------------------------------------------------------------- encoding

def _nearest_even(x: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Code of the grid value nearest to x >= 0, ties to the even code.

    ``grid`` lists the non-negative finite values in code order (code == index,
    values increasing).  x above the largest value maps to the largest code.
    """
    x = np.asarray(x, dtype=np.float64)
    top = len(grid) - 1
    hi = np.searchsorted(grid, x, side="left")          # grid[hi-1] < x <= grid[hi]
    hi = np.clip(hi, 1, top)
    lo = hi - 1
    mid = (grid[lo] + grid[hi]) / 2.0                   # exact: few significant bits
    code = np.where(x < mid, lo, hi)
    tie = x == mid
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(x >= grid[top], top, code)
    code = np.where(x <= 0, 0, code)
    return code.astype(np.uint8)


_E4M3_POS = E4M3_TABLE[:0x7F]     # codes 0x00..0x7E: 0 .. 448
_E2M1_POS = E2M1_TABLE[:8]        # codes 0x0..0x7:   0 .. 6


def e4m3_encode(v) -> np.ndarray:
    """Round v (float64, finite) to E4M3, ties to even; magnitudes above 448 clamp."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_even(np.abs(v), _E4M3_POS)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def e2m1_encode(v) -> np.ndarray:
    """Round v (float64, finite) to E2M1 (4-bit code), ties to even; clamps at 6."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_even(np.abs(v), _E2M1_POS)
    sign = np.signbit(v).astype(np.uint8) << 3
    return (mag | sign).astype(np.uint8)


# ---------------------------------------------------------------- block scale

def block_exponent(amax, qmax: float) -> np.ndarray:
    """Smallest integer e with amax <= qmax * 2^e (0 where amax == 0), clamped to
    the E8M0 range [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    _, xa = np.frexp(safe)
    _, xq = np.frexp(qmax)
    e = (xa - xq).astype(np.int64)
    # Fix up to the exact smallest exponent (at most a couple of steps each way).
    for _ in range(3):
        e = np.where(safe > np.ldexp(qmax, e), e + 1, e)
    for _ in range(3):
        e = np.where(safe <= np.ldexp(qmax, e - 1), e - 1, e)
    e = np.where(pos, e, 0)
    return np.clip(e, -127, 127)


def _quantize_groups(g: np.ndarray, fmt: str):
    """g [n, 32] float64 -> (codes uint8 [n, 32], scale bytes uint8 [n])."""
    qmax = E4M3_MAX if fmt == "e4m3" else E2M1_MAX
    e = block_exponent(np.abs(g).max(axis=-1), qmax)
    scaled = np.ldexp(g, -e[:, None])
    codes = e4m3_encode(scaled) if fmt == "e4m3" else e2m1_encode(scaled)
    return codes, (e + 127).astype(np.uint8)


def quantize_blocks(v, fmt: str):
    """Quantise v [..., K] (K % 32 == 0) in groups of 32 along the last axis.

    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32]).  fmt is
    "e4m3" or "e2m1" (E2M1 codes are returned one per byte, unpacked).
    Groups are independent; large inputs are cut into chunks of groups that
    run on a thread pool (numpy releases the GIL), with identical results.
    """
    v = np.asarray(v)
    K = v.shape[-1]
    assert K % GROUP == 0
    g = v.reshape(-1, GROUP)
    n = g.shape[0]
    codes = np.empty((n, GROUP), np.uint8)
    sf = np.empty(n, np.uint8)
    chunk = 1 << 16

    def run(i):
        sl = slice(i, min(i + chunk, n))
        codes[sl], sf[sl] = _quantize_groups(g[sl].astype(np.float64), fmt)

    starts = range(0, n, chunk)
    if n > chunk:
        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(run, starts))
    else:
        for i in starts:
            run(i)
    return codes.reshape(v.shape), sf.reshape(*v.shape[:-1], K // GROUP)


def dequantize_blocks(codes, sf, fmt: str) -> np.ndarray:
    """Inverse of quantize_blocks: code value * 2^(b - 127), float64 [..., K]."""
    codes = np.asarray(codes)
    table = E4M3_TABLE if fmt == "e4m3" else E2M1_TABLE
    vals = table[codes.astype(np.int64)]
    K = vals.shape[-1]
    g = vals.reshape(*vals.shape[:-1], K // GROUP, GROUP)
    g = g * e8m0_value(sf)[..., None]
    return g.reshape(vals.shape)


# ---------------------------------------------------------------- FP4 packing

def pack_e2m1(codes) -> np.ndarray:
    """Two E2M1 codes per byte along the last axis: element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_e2m1(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------- BF16

def bf16_bits(f32) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); returns uint16 bits.

    Written out on the bit pattern: keep the top 16 bits, add one unit in the
    last kept place when the dropped half exceeds one half, or equals one half
    and the kept part is odd.  NaN stays NaN.
    """
    f = np.ascontiguousarray(f32, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep = u >> 16
    drop = u & 0xFFFF
    up = (drop > 0x8000) | ((drop == 0x8000) & ((keep & 1) == 1))
    r = (keep + up.astype(np.uint64)).astype(np.uint32)
    nan = np.isnan(f)
    r = np.where(nan, (keep | 0x40).astype(np.uint32), r)
    return r.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """BF16 bit patterns -> float32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
