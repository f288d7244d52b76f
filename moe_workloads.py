"""Seeded synthetic inputs for the top-k MoE layer workloads.

This module is shared by the CPU oracle's tests, the GPU tests, the smoke check
and the benchmark.  It only draws random numbers and lays them out; it contains
none of the layer's arithmetic (no routing, no quantisation, no GEMM).  Both the
oracle and the GPU path quantise the BF16 weights produced here on their own.

Streams: every tensor has its own ``numpy.random.Generator(SFC64(SeedSequence(
[seed, key...])))`` stream, so tensors can be generated independently and in
parallel, and a sample of experts can be regenerated without the rest.

  logits  [T, E] float32 ~ N(0, 1)                       key (1,)
  x       [T, H] bf16    ~ N(0, 1)                        key (2,)
  W13[e]  [2I, H] bf16   ~ 0.02 * N(0, 1), gate rows then up rows   key (3, e)
  W2[e]   [H, I]  bf16   ~ 0.02 * N(0, 1)                 key (4, e)
  zipf permutation for the skewed workload                key (5,)
  external top-k ids (random distinct experts per token)  key (6,)

Values are drawn as float32 and rounded to BF16 by torch's cast (round to
nearest even).  BF16 tensors are returned as uint16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

SOFTMAX = 0
SIGMOID = 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int           # tokens
    H: int           # hidden
    I: int           # intermediate (per gate / up half)
    E: int           # experts
    topk: int
    score_fn: int = SOFTMAX   # 0 softmax, 1 sigmoid
    renorm: int = 1
    zipf_s: float = 0.0       # >0: bias logits so expert popularity follows Zipf(s)
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.topk

    def flops(self) -> float:
        """Algorithmic FLOPs of one layer call: GEMM1 4RIH + GEMM2 2RHI."""
        return 6.0 * self.R * self.H * self.I

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T)


# The five workloads the layer is specified on (one GPU's share of the work).
WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=256, I=128, E=8, topk=2),
    "decode": Workload("decode", T=8, H=2048, I=512, E=256, topk=8),
    "dsv3_prefill": Workload("dsv3_prefill", T=4096, H=7168, I=2048, E=32, topk=8),
    "dsv3_skewed": Workload("dsv3_skewed", T=4096, H=7168, I=2048, E=32, topk=8, zipf_s=1.2),
    "full256": Workload("full256", T=8192, H=7168, I=2048, E=256, topk=8, score_fn=SIGMOID),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, *key])))


def _normal_f32(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> BF16 bit patterns (uint16), rounded to nearest even by torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def zipf_bias(w: Workload) -> np.ndarray:
    """Per-expert logit bias 2*ln p(rank), p = Zipf(s) over E ranks, ranks permuted."""
    ranks = np.arange(1, w.E + 1, dtype=np.float64)
    p = ranks ** (-w.zipf_s)
    p /= p.sum()
    perm = _rng(w.seed, 5).permutation(w.E)
    return (2.0 * np.log(p[perm])).astype(np.float32)


def gen_logits(w: Workload) -> np.ndarray:
    z = _normal_f32(_rng(w.seed, 1), (w.T, w.E))
    if w.zipf_s > 0:
        z += zipf_bias(w)[None, :]
    return z


def gen_x(w: Workload) -> np.ndarray:
    return to_bf16_bits(_normal_f32(_rng(w.seed, 2), (w.T, w.H)))


def gen_expert_w13(w: Workload, e: int) -> np.ndarray:
    """[2I, H] BF16 bits; rows [0, I) gate, rows [I, 2I) up; K (= H) contiguous."""
    return to_bf16_bits(_normal_f32(_rng(w.seed, 3, e), (2 * w.I, w.H), 0.02))


def gen_expert_w2(w: Workload, e: int) -> np.ndarray:
    """[H, I] BF16 bits; K (= I) contiguous."""
    return to_bf16_bits(_normal_f32(_rng(w.seed, 4, e), (w.H, w.I), 0.02))


def gen_weights(w: Workload, experts=None, threads: int | None = None):
    """BF16 W13 [n, 2I, H] and W2 [n, H, I] for the listed experts (default: all)."""
    experts = list(range(w.E)) if experts is None else list(experts)
    n = len(experts)
    w13 = np.empty((n, 2 * w.I, w.H), np.uint16)
    w2 = np.empty((n, w.H, w.I), np.uint16)

    def one(i):
        w13[i] = gen_expert_w13(w, experts[i])
        w2[i] = gen_expert_w2(w, experts[i])

    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(n)))
    return w13, w2


def gen_external_topk(w: Workload, mask_frac: float = 0.0):
    """Router output supplied by a caller: distinct random experts per token.

    Ids are int32 [T, k]; a fraction ``mask_frac`` of entries is set to -1
    (masked slots).  Weights are float32 [T, k] ~ U(0, 1).
    """
    rng = _rng(w.seed, 6)
    keys = rng.random((w.T, w.E))
    idx = np.argsort(keys, axis=1, kind="stable")[:, : w.topk].astype(np.int32)
    wt = rng.random((w.T, w.topk), dtype=np.float32)
    if mask_frac > 0:
        m = rng.random((w.T, w.topk)) < mask_frac
        idx[m] = -1
    return idx, wt


def tiny_shapes():
    """Small random shapes used for exhaustive CPU checks."""
    out = []
    for T in (1, 3, 17):
        for E, k in ((1, 1), (2, 1), (2, 2), (5, 2)):
            for H, I in ((32, 32), (64, 32), (32, 64)):
                out.append(Workload(f"t{T}e{E}k{k}h{H}i{I}", T=T, H=H, I=I, E=E, topk=k))
    return out
