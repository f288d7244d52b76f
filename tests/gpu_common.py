"""Shared helpers of the GPU parity tests: device setup of a workload through
the library, oracle expectations on the same seeded inputs, and the tolerance
checks of the layer.

Tolerances (floating point only; integer outputs are compared exactly):
  y     max|y - y_ref| <= 2e-2 * max|y_ref| and
        sum|y - y_ref| / sum|y_ref| <= 5e-3 (normalised L1 error)
  hq    the E4M3 intermediates, compared as values (code x scale):
          - at most 0.1 % of them differ;
          - a differing value is at most one E4M3 grid step from the reference,
            measured on the grid of the larger of the two group scales;
          - (with block-FP8 weights, whose float32 scales move in their last
            bits with each group's largest value, the codes are compared
            instead, and the scales must agree to a relative 1e-4)
          - the only exception is a value whose own rounding error bound
            allows more: the GPU and the reference each round a dot product of
            K FP8 x FP4 products in FP32, in different orders, so each
            accumulator (gate g, up u) may differ by (c + gamma_n) *
            sum_k |a_k b_k|: c is the matrix instruction's own accumulation
            error per 128 products (measured: MFMA_FP8_FP4_REL, MFMA_BF16_REL;
            the FP8 instructions do not sum in FP32), gamma_n = n u / (1 - n u)
            (u = 2^-24) is Higham's bound for the FP32 sum of the n partials
            (K/128 blocks, plus the narrow kernel's four per-wave sums), which
            reaches h = silu(g) * u * w through |w| (L dg (|u| + du) +
            |silu(g)| du) with L = max |silu'| < 1.1, plus a few FP32 roundings
            of silu and the products; the two values may then differ by that
            bound plus one grid step.  Values that are small through
            cancellation (|h| far below sum_k |a_k b_k|) are the only ones it
            lets move by more than a step; at most 1e-4 of the values may use
            it, and each is reported.
  topk_w  relative 4e-6 (float32 exp/divide against the float64 reference)

Every check prints its margins (the y error ratios against their limits, the
fraction of differing hq values, the largest distance in grid steps and the
number of values beyond one step).
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import moe_workloads as W
from oracle import codecs as C
from oracle import moe_ref as M

DEV = "cuda"

# Accumulation error of one matrix instruction (128 products) as a fraction of
# sum |a b|, measured by tests/probes/mfma_precision and asserted by
# tests/test_gpu_instruction_precision.py: over random codes the FP8 x FP4 scaled
# MFMA reached 2^-13.8 (the FP8 x FP8 one 2^-12.6), four BF16 MFMAs over widened
# E4M3 values 2^-21.8 (1000 random tiles).
MFMA_FP8_FP4_REL = 2.0 ** -13
MFMA_BF16_REL = 2.0 ** -20


def lib():
    import mixture_experts_layer_topk_amd as m
    return m


def to_dev(a: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def bf16_dev(bits: np.ndarray):
    return to_dev(bits.view(np.int16), torch.bfloat16)


@functools.lru_cache(maxsize=320)
def _oracle_expert(seed: int, H: int, I: int, e: int):
    w = W.Workload("weights", T=1, H=H, I=I, E=e + 1, topk=1, seed=seed)
    q13, s13 = M.pack_weights(W.gen_expert_w13(w, e))
    q2, s2 = M.pack_weights(W.gen_expert_w2(w, e))
    return q13, s13, q2, s2


def oracle_expert(w: W.Workload, e: int):
    """Oracle-packed weights of expert e (from the same seeded BF16 values; the
    weights depend on the seed and shapes only, so workloads that differ in their
    tokens or routing share them)."""
    return _oracle_expert(w.seed, w.H, w.I, int(e))


def prefetch_oracle_experts(w: W.Workload, experts=None, threads: int = 16):
    """Pack the listed experts' weights with the oracle on a thread pool (numpy
    releases the GIL in the heavy steps), so later serial lookups hit the cache."""
    experts = range(w.E) if experts is None else experts
    with ThreadPoolExecutor(min(threads, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda e: oracle_expert(w, e), experts))


class LazyExperts:
    """Indexable by expert id, packing experts with the oracle on first use."""

    def __init__(self, w, field):
        self.w, self.field = w, field

    def __getitem__(self, e):
        return oracle_expert(self.w, int(e))[self.field]

    def __len__(self):
        return self.w.E


def oracle_weights(w):
    return [LazyExperts(w, i) for i in range(4)]


class DeviceLayer:
    """A workload's inputs on the GPU, weights packed by the library."""

    def __init__(self, w: W.Workload, external_topk=None):
        m = lib()
        self.w = w
        self.x_np = W.gen_x(w)
        self.logits_np = W.gen_logits(w)
        self.x = bf16_dev(self.x_np)
        self.logits = to_dev(self.logits_np)
        self.topk_idx = self.topk_w = None
        if external_topk is not None:
            self.topk_idx = to_dev(external_topk[0])
            self.topk_w = to_dev(external_topk[1])
        self.w13q = torch.empty((w.E, 2 * w.I, w.H // 2), dtype=torch.uint8, device=DEV)
        self.w13sf = torch.empty((w.E, 2 * w.I, w.H // 32), dtype=torch.uint8, device=DEV)
        self.w2q = torch.empty((w.E, w.H, w.I // 2), dtype=torch.uint8, device=DEV)
        self.w2sf = torch.empty((w.E, w.H, w.I // 32), dtype=torch.uint8, device=DEV)
        gen = lambda e: (W.gen_expert_w13(w, e), W.gen_expert_w2(w, e))
        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            for e, (b13, b2) in enumerate(ex.map(gen, range(w.E))):
                q, s = m.pack_weights(bf16_dev(b13))
                self.w13q[e], self.w13sf[e] = q, s
                q, s = m.pack_weights(bf16_dev(b2))
                self.w2q[e], self.w2sf[e] = q, s
        # per-row scales (compared with the oracle) and the K-step-major copies the layer takes
        self.w13sf_k = m.scales_kmajor(self.w13sf, w.H)
        self.w2sf_k = m.scales_kmajor(self.w2sf, w.I)
        self.d = m.dims(w.T, w.H, w.I, w.E, w.topk, w.score_fn, w.renorm)
        self.ws = m.new_workspace(self.d)
        self._staged = None

    def staged(self):
        """The weight codes in the staged layout (made on first use)."""
        if self._staged is None:
            m = lib()
            self._staged = (m.stage_weights(self.w13q, True), m.stage_weights(self.w2q, False))
        return self._staged

    def forward(self, use_logits=True, flags=0, staged=False):
        """One layer call; staged: with the staged weight codes (FLAG_W_STAGED)."""
        m = lib()
        w13q, w2q = self.staged() if staged else (self.w13q, self.w2q)
        if staged:
            flags |= m.FLAG_W_STAGED
        if self.topk_idx is not None and not use_logits:
            y = m.forward(self.d, self.x, w13q, self.w13sf_k, w2q, self.w2sf_k, self.ws,
                          topk_idx=self.topk_idx, topk_w=self.topk_w, flags=flags)
        else:
            y = m.forward(self.d, self.x, w13q, self.w13sf_k, w2q, self.w2sf_k, self.ws,
                          logits=self.logits, flags=flags)
        torch.cuda.synchronize()
        status = int(m.intermediates(self.d, self.ws)["status"].item())
        assert status == 0, f"a wait inside the layer gave up (status {status})"
        return y

    def intermediates(self):
        return {k: v.cpu().numpy() for k, v in lib().intermediates(self.d, self.ws).items()}


def y_bits(y: torch.Tensor) -> np.ndarray:
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def check_y(y_gpu_bits, y_ref_bits, rows=None, label="y"):
    a = C.bf16_value(y_gpu_bits).astype(np.float64)
    b = C.bf16_value(y_ref_bits).astype(np.float64)
    if rows is not None:
        a, b = a[rows], b[rows]
    assert np.isfinite(a).all()
    err = np.abs(a - b)
    mx = np.abs(b).max()
    l1 = err.sum() / max(np.abs(b).sum(), 1e-30)
    print(f"    {label}: {a.shape[0]} rows, max|dy|/max|y| = {err.max() / mx:.3e} (limit 2e-2), "
          f"normalised L1 = {l1:.3e} (limit 5e-3)", flush=True)
    assert err.max() <= 2e-2 * mx, f"max err {err.max()} vs {2e-2 * mx}"
    assert l1 <= 5e-3, f"normalised L1 {l1}"
    return err.max() / mx, l1


def e4m3_position(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Signed position of value v on the E4M3 grid of scale s, in grid steps from
    zero: the code's magnitude index (8 * biased exponent + mantissa, 0..126) for
    grid values, linear in between.  Positions of two values of one grid differ by
    the number of grid steps between them."""
    x = np.abs(v) / s
    sub = x < 2.0 ** -6
    ex = np.floor(np.log2(np.where(sub, 1.0, x)))
    pos = np.where(sub, x * 2.0 ** 9, 8.0 * (ex + 7) + (x / np.ldexp(1.0, ex.astype(int)) - 1.0) * 8.0)
    return np.sign(v) * pos


def check_hq(hq_g, hsf_g, hq_r, hsf_r, max_frac=1e-3, bound=None, max_beyond=1e-4, label="hq",
             block=32):
    """hq against the reference (see the module docstring).  bound(rows, cols)
    returns the accumulation-order bound of |h_gpu - h_ref| for those elements
    (float64); without it no value may be more than one grid step away.

    block=32: UE8M0 scale bytes per 32 elements, compared in value space (a scale
    that flips by a factor 2 changes every code of its group).  block=128: float32
    scales per 128 elements (block-FP8 weights): a scale is max|h| / 448, so it
    moves in its last bits with the group's largest value, which moves every value
    and no code; there the codes are compared (at most max_frac differ, each by one
    code step unless its bound allows more) and the scales must agree to a relative
    1e-4."""
    n = hq_g.size
    if block == 32:
        a = C.dequantize_blocks(hq_g, hsf_g, "e4m3")
        b = C.dequantize_blocks(hq_r, hsf_r, "e4m3")
        sc_g, sc_r = C.e8m0_value(hsf_g), C.e8m0_value(hsf_r)
        diff = a != b
    else:
        sc_g, sc_r = np.asarray(hsf_g, np.float64), np.asarray(hsf_r, np.float64)
        rel = np.abs(sc_g - sc_r) / np.maximum(sc_r, 1e-300)
        print(f"    {label}: float32 scales agree to a relative {rel.max():.2e} (limit 1e-4)", flush=True)
        assert rel.max() <= 1e-4, f"scales differ by a relative {rel.max():.2e}"
        a = C.E4M3_TABLE[hq_g.astype(np.int64)] * np.repeat(sc_g, block, -1)
        b = C.E4M3_TABLE[hq_r.astype(np.int64)] * np.repeat(sc_r, block, -1)
        diff = hq_g != hq_r
    nd = int(diff.sum())
    frac = nd / n if n else 0.0
    max_steps, beyond = 0.0, 0
    if nd:
        s = np.maximum(np.repeat(sc_g, block, -1), np.repeat(sc_r, block, -1))
        r, c = np.nonzero(diff)
        sd = s[r, c]
        if block == 32:
            steps = np.abs(e4m3_position(a[r, c], sd) - e4m3_position(b[r, c], sd))
        else:
            # code steps: the magnitude codes 0x00..0x7E are in value order
            def signed(code):
                code = code.astype(np.int64)
                return np.where(code & 0x80, -(code & 0x7F), code & 0x7F)
            steps = np.abs(signed(hq_g[r, c]) - signed(hq_r[r, c])).astype(np.float64)
        max_steps = float(steps.max())
        far = steps > 1.0 + 1e-9
        beyond = int(far.sum())
        if beyond:
            rr, cc = r[far], c[far]
            big = np.maximum(np.abs(a[rr, cc]), np.abs(b[rr, cc]))
            pos = e4m3_position(big, sd[far])
            # one grid step at the larger value: 2^-9 s below 2^-6 s, else 2^(e-3) s
            step = np.where(pos < 8.0, 2.0 ** -9, np.ldexp(1.0, (np.floor(pos / 8.0) - 7 - 3).astype(int))) * sd[far]
            if bound is None:
                lim = np.zeros_like(step)
            else:
                lim = bound(rr, cc)
            bad = np.abs(a[rr, cc] - b[rr, cc]) > (lim + step) * (1 + 1e-9)
            lines = [f"row {i} col {j}: gpu code {hq_g[i, j]:#04x} sf {hsf_g[i, j // block]} = {a[i, j]:.6g}, "
                     f"ref code {hq_r[i, j]:#04x} sf {hsf_r[i, j // block]} = {b[i, j]:.6g}, "
                     f"bound {l:.3g} + step {st:.3g}"
                     for i, j, l, st in list(zip(rr, cc, lim, step))[:12]]
            print(f"    {label}: {beyond} value(s) beyond one grid step:\n      " + "\n      ".join(lines),
                  flush=True)
            assert not bad.any(), f"{int(bad.sum())} hq values differ beyond their accumulation bound"
    what = "values" if block == 32 else "codes"
    print(f"    {label}: {n} {what}, {nd} differ ({frac:.2e}, limit {max_frac:.0e}); largest distance "
          f"{max_steps:.3g} grid steps; {beyond} beyond one step (limit {max_beyond:.0e} of the values)",
          flush=True)
    assert frac <= max_frac, f"{frac:.2e} of hq differ"
    assert beyond <= max_beyond * n, f"{beyond} hq values beyond one grid step"
    return frac


def accumulation_rel(K: int, instr_rel: float) -> float:
    """Bound on |acc_gpu - acc_exact| / sum_k |a_k b_k| for a K-long dot product
    formed as K/128 instruction partials (each within instr_rel) summed in FP32 with
    up to four more partial sums, plus the reference's own rounding to FP32."""
    u32 = 2.0 ** -24
    n = K // 128 + 5
    return instr_rel + n * u32 / (1 - n * u32)


def make_hq_bound(ref, pairs, w13q, w13sf, topk: int, I: int):
    """bound(rows, cols) for check_hq: compared row i is pair pairs[i] = t*topk + j of
    the reference ``ref`` (an oracle forward); w13q/w13sf index the oracle's packed
    weights by expert.  Recomputes g, u and sum_k |a_k b_k| of each asked element in
    float64 from the dequantised operands."""
    u32 = 2.0 ** -24

    def bound(rows, cols):
        out = np.empty(len(rows))
        for n, (i, c) in enumerate(zip(rows, cols)):
            f = int(pairs[i])
            t, j = f // topk, f % topk
            e = int(ref["topk_idx"][t, j])
            wt = float(ref["topk_w"][t, j])
            a = C.dequantize_blocks(ref["xq"][t:t + 1], ref["xsf"][t:t + 1], "e4m3")[0]
            K = a.size
            rows13 = C.dequantize_blocks(C.unpack_e2m1(w13q[e][[c, I + c]]), w13sf[e][[c, I + c]], "e2m1")
            g, u = float(a @ rows13[0]), float(a @ rows13[1])
            gamma = accumulation_rel(K, MFMA_FP8_FP4_REL)
            dg = gamma * float(np.abs(a) @ np.abs(rows13[0]))
            du = gamma * float(np.abs(a) @ np.abs(rows13[1]))
            silu = g / (1.0 + np.exp(-g)) if g > -700 else 0.0
            h = silu * u * wt
            out[n] = abs(wt) * (1.1 * dg * (abs(u) + du) + (abs(silu) + 1.1 * dg) * du) + 16 * u32 * abs(h)
        return out

    return bound


def check_bucketize(inter, idx_ref, E):
    """Counts/offsets exact; each expert segment holds exactly its pairs; slot_of inverse."""
    T, k = idx_ref.shape
    counts = np.bincount(idx_ref[idx_ref >= 0].reshape(-1), minlength=E)
    assert np.array_equal(inter["counts"], counts)
    off = np.concatenate([[0], np.cumsum(counts)])
    assert np.array_equal(inter["offsets"], off)
    n = off[-1]
    src = inter["slot_src"][:n]
    flat = idx_ref.reshape(-1)
    for e in range(E):
        seg = np.sort(src[off[e]:off[e + 1]])
        assert np.array_equal(seg, np.nonzero(flat == e)[0]), f"expert {e} segment"
    so = inter["slot_of"].reshape(-1)
    valid = flat >= 0
    assert np.all(so[~valid] == -1)
    assert np.array_equal(src[so[valid]], np.nonzero(valid)[0])
