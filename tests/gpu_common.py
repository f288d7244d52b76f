"""Shared helpers of the GPU parity tests: device setup of a workload through
the library, oracle expectations on the same seeded inputs, and the tolerance
checks of the layer.

Tolerances (floating point only; integer outputs are compared exactly):
  y     max|y - y_ref| <= 2e-2 * max|y_ref| and
        sum|y - y_ref| / sum|y_ref| <= 5e-3 (normalised L1 error)
  hq    at most 0.1 % of the E4M3 intermediates differ, each by at most one
        E4M3 step at the larger of the two values, or by at most 2^-12 of its
        group's range 448 * scale (FP32 accumulation order and the exp of SiLU
        may move a value across a rounding boundary; the FP32 accumulation
        error of a dot product scales with the sum of |products|, so values
        that are small through cancellation can move by a few codes)
  topk_w  relative 4e-6 (float32 exp/divide against the float64 reference)
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


@functools.lru_cache(maxsize=64)
def oracle_expert(w: W.Workload, e: int):
    """Oracle-packed weights of expert e (from the same seeded BF16 values)."""
    q13, s13 = M.pack_weights(W.gen_expert_w13(w, e))
    q2, s2 = M.pack_weights(W.gen_expert_w2(w, e))
    return q13, s13, q2, s2


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

    def forward(self, use_logits=True, flags=0):
        m = lib()
        if self.topk_idx is not None and not use_logits:
            y = m.forward(self.d, self.x, self.w13q, self.w13sf_k, self.w2q, self.w2sf_k, self.ws,
                          topk_idx=self.topk_idx, topk_w=self.topk_w, flags=flags)
        else:
            y = m.forward(self.d, self.x, self.w13q, self.w13sf_k, self.w2q, self.w2sf_k, self.ws,
                          logits=self.logits, flags=flags)
        torch.cuda.synchronize()
        status = int(m.intermediates(self.d, self.ws)["status"].item())
        assert status == 0, f"a wait inside the layer gave up (status {status})"
        return y

    def intermediates(self):
        return {k: v.cpu().numpy() for k, v in lib().intermediates(self.d, self.ws).items()}


def y_bits(y: torch.Tensor) -> np.ndarray:
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def check_y(y_gpu_bits, y_ref_bits, rows=None):
    a = C.bf16_value(y_gpu_bits).astype(np.float64)
    b = C.bf16_value(y_ref_bits).astype(np.float64)
    if rows is not None:
        a, b = a[rows], b[rows]
    assert np.isfinite(a).all()
    err = np.abs(a - b)
    mx = np.abs(b).max()
    l1 = err.sum() / max(np.abs(b).sum(), 1e-30)
    assert err.max() <= 2e-2 * mx, f"max err {err.max()} vs {2e-2 * mx}"
    assert l1 <= 5e-3, f"normalised L1 {l1}"
    return err.max() / mx, l1


def e4m3_step(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """One E4M3 grid step at value |v| for scale s (subnormal step below 2^-6 s)."""
    mag = np.abs(v) / s
    ex = np.floor(np.log2(np.maximum(mag, 2.0 ** -6)))
    return np.ldexp(1.0, (ex - 3).astype(int)) * s


def check_hq(hq_g, hsf_g, hq_r, hsf_r, max_frac=1e-3):
    a = C.dequantize_blocks(hq_g, hsf_g, "e4m3")
    b = C.dequantize_blocks(hq_r, hsf_r, "e4m3")
    diff = a != b
    frac = diff.mean() if diff.size else 0.0
    assert frac <= max_frac, f"{frac:.2e} of hq differ"
    if diff.any():
        s = np.maximum(np.repeat(C.e8m0_value(hsf_g), 32, -1), np.repeat(C.e8m0_value(hsf_r), 32, -1))
        big = np.maximum(np.abs(a), np.abs(b))
        step = e4m3_step(big, s)
        tol = np.maximum(step, 448.0 * s * 2.0 ** -12)
        bad = diff & (np.abs(a - b) > tol * (1 + 1e-12))
        if bad.any():
            r, c = np.nonzero(bad)
            lines = [f"row {i} col {j}: gpu code {hq_g[i, j]:#04x} sf {hsf_g[i, j // 32]} = {a[i, j]:.6g}, "
                     f"ref code {hq_r[i, j]:#04x} sf {hsf_r[i, j // 32]} = {b[i, j]:.6g}"
                     for i, j in list(zip(r, c))[:12]]
            raise AssertionError(f"{bad.sum()} hq values differ beyond tolerance "
                                 f"(rows {np.unique(r)[:20]}):\n" + "\n".join(lines))
    return frac


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
