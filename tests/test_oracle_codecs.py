"""Pins for oracle/codecs.py: format definitions, torch casts, invariants.

These do not compare the oracle with itself: decode tables are checked against
torch's float8 views and the OCP value sets, E4M3 rounding against torch's
float32 -> float8_e4m3fn cast over every finite BF16 value, E2M1 rounding and
the block exponent against exact rational search, BF16 rounding against torch.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs as C
from tests import brute_force as BF


# ------------------------------------------------------------ decode tables

def test_e4m3_table_matches_torch_view():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan_o, nan_t = np.isnan(C.E4M3_TABLE), np.isnan(t)
    assert (nan_o == nan_t).all()
    assert nan_o.sum() == 2 and nan_o[0x7F] and nan_o[0xFF]
    assert np.array_equal(C.E4M3_TABLE[~nan_o], t[~nan_t])
    # signed zero
    assert math.copysign(1, C.E4M3_TABLE[0x80]) < 0


def test_e4m3_landmarks():
    assert C.E4M3_TABLE[0x7E] == 448.0                  # largest finite
    assert C.E4M3_TABLE[0x01] == 2.0 ** -9              # smallest subnormal
    assert C.E4M3_TABLE[0x08] == 2.0 ** -6              # smallest normal
    assert C.E4M3_TABLE[0x38] == 1.0
    assert np.all(np.diff(C.E4M3_TABLE[:0x7F]) > 0)     # monotone in code order


def test_e2m1_table_is_ocp_value_set():
    assert C.E2M1_TABLE[:8].tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert C.E2M1_TABLE[8:].tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def test_e8m0_matches_torch_view():
    b = np.arange(256)
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    o = C.e8m0_value(b)
    assert np.isnan(o[255]) and np.isnan(t[255])
    assert np.array_equal(o[:255], t[:255])
    assert o[127] == 1.0 and o[0] == 2.0 ** -127 and o[254] == 2.0 ** 127


# ------------------------------------------------------------ encoders

def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_e4m3_encode_matches_torch_for_every_bf16_in_range():
    f = _all_finite_bf16()
    f = f[np.abs(f) <= 448.0]
    ours = C.e4m3_encode(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_matches_torch_random_fp32():
    rng = np.random.default_rng(1)
    f = (rng.standard_normal(2_000_000) * np.exp2(rng.integers(-14, 9, 2_000_000))).astype(np.float32)
    f = f[np.abs(f) <= 448.0]
    # include exact midpoints between neighbouring codes (ties)
    vals = C.E4M3_TABLE[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    f = np.concatenate([f, mids, -mids])
    ours = C.e4m3_encode(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_clamps_above_max():
    assert C.e4m3_encode(np.array([449.0, 1e6, -1e6])).tolist() == [0x7E, 0x7E, 0xFE]


def test_e2m1_encode_matches_rational_search():
    xs = [k / 64 for k in range(-64 * 7, 64 * 7 + 1)] + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0]
    ours = C.e2m1_encode(np.array(xs))
    for x, c in zip(xs, ours):
        assert c == BF.e2m1_round(Fraction(x), math.copysign(1, x) < 0), x


def test_e2m1_ties_go_to_even_codes():
    # midpoints: 0.25 (0|0.5), 0.75 (0.5|1), 1.25, 1.75, 2.5, 3.5, 5
    got = C.e2m1_encode(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])).tolist()
    assert got == [0, 2, 2, 4, 4, 6, 6]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    u = rng.integers(0, 1 << 32, 3_000_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = C.bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7FFFFF], np.uint32).view(np.float32)
    assert np.array_equal(C.bf16_bits(ties),
                          torch.from_numpy(ties).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------ block exponent / quantiser

@pytest.mark.parametrize("q", [448.0, 6.0])
def test_block_exponent_matches_rational_search(q):
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000)))
    amax = np.concatenate([amax, [q, q * 2, q / 2, q * 0.999, 1.0, 1.75, 1.5, 2.0 ** -140, 0.0]])
    ours = C.block_exponent(amax, q)
    for a, e in zip(amax, ours):
        assert e == BF.min_exponent(Fraction(float(a)), Fraction(q)), a


def _groups(seed, n=4096):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((n, 32)) * np.exp2(rng.integers(-20, 20, (n, 1)))
    g = g.astype(np.float32).astype(np.float64)
    g[0] = 0.0
    g[1, :] = 0.0
    g[1, 5] = -3.0
    return g


@pytest.mark.parametrize("fmt,q", [("e4m3", 448.0), ("e2m1", 6.0)])
def test_quantiser_scale_is_minimal(fmt, q):
    g = _groups(4)
    codes, sf = C.quantize_blocks(g, fmt)
    s = np.ldexp(1.0, sf[:, 0].astype(int) - 127)
    amax = np.abs(g).max(1)
    nz = amax > 0
    r = amax[nz] / s[nz]
    assert np.all(r <= q) and np.all(r > q / 2)
    assert np.all(sf[~nz, 0] == 127)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantiser_error_at_most_half_step(fmt):
    g = _groups(5)
    codes, sf = C.quantize_blocks(g, fmt)
    dq = C.dequantize_blocks(codes, sf, fmt)
    table = (C.E4M3_TABLE[:0x7F] if fmt == "e4m3" else C.E2M1_TABLE[:8])
    s = np.ldexp(1.0, sf.astype(int) - 127)[:, :1]
    x = np.abs(g) / s
    # local grid spacing around x
    hi = np.clip(np.searchsorted(table, x), 1, len(table) - 1)
    step = table[hi] - table[hi - 1]
    assert np.all(np.abs(dq - g) / s <= step / 2 + 0.0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantiser_sign_symmetry(fmt):
    g = _groups(6)
    c1, s1 = C.quantize_blocks(g, fmt)
    c2, s2 = C.quantize_blocks(-g, fmt)
    sign = 0x80 if fmt == "e4m3" else 0x8
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1 ^ sign, c2)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("m", [-5, 1, 7])
def test_quantiser_power_of_two_equivariance(fmt, m):
    g = _groups(7)
    c1, s1 = C.quantize_blocks(g, fmt)
    c2, s2 = C.quantize_blocks(np.ldexp(g, m), fmt)
    nz = np.abs(g).max(1) > 0
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2[nz].astype(int), s1[nz].astype(int) + m)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantiser_idempotent(fmt):
    g = _groups(8)
    c1, s1 = C.quantize_blocks(g, fmt)
    d1 = C.dequantize_blocks(c1, s1, fmt)
    c2, s2 = C.quantize_blocks(d1, fmt)
    d2 = C.dequantize_blocks(c2, s2, fmt)
    assert np.array_equal(d1, d2)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantiser_matches_brute_force_groups(fmt):
    g = _groups(9, n=200)
    codes, sf = C.quantize_blocks(g, fmt)
    for r in range(g.shape[0]):
        c, s = BF.quant_group(g[r].tolist(), fmt)
        assert s == sf[r, 0]
        assert list(codes[r]) == c


def test_fp4_pack_roundtrip_and_nibble_order():
    rng = np.random.default_rng(10)
    c = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    p = C.pack_e2m1(c)
    assert p.shape == (7, 32)
    assert np.array_equal(p[:, 0] & 0xF, c[:, 0]) and np.array_equal(p[:, 0] >> 4, c[:, 1])
    assert np.array_equal(C.unpack_e2m1(p), c)
