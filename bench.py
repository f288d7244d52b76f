"""Benchmark of the fused FP8 x FP4 top-k MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one moe_forward call (route -> bucketise -> quantise -> GEMM1 +
SwiGLU*w -> GEMM2 -> combine) on inputs already resident in HBM.  The default
workload is the DeepSeek-V3-like one-GPU expert share (T=4096, H=7168,
I=2048, E=32, top-8).  Prints one JSON line.

Roofline: per-stage times come from HIP events the library records on the
launch stream at stage boundaries inside the timed region; GEMM1 (two thirds of
the FLOPs) is reported against the dense FP8-rate MFMA peak.  cpu_baseline: the
CPU oracle timed on a bounded sample of tokens of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_FP8_TFLOPS = 5000.0      # MI355X dense FP8-rate MFMA (FP8 x FP4 issues at this rate)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--cpu-sample-tokens", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before the timed steps, copy a buffer of this many MiB once (a "
                         "plain copy kernel of known size, to calibrate traffic counters)")
    ap.add_argument("--flush-mb", type=int, default=0,
                    help="write this many MiB between steps (outside the timed events) to "
                         "evict the last-level cache; 0 = off")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the timing needs (events on the launch stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def setup_device(w, m, torch):
    import moe_workloads as W
    from concurrent.futures import ThreadPoolExecutor

    dev = "cuda"
    x = torch.from_numpy(W.gen_x(w).view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(W.gen_logits(w)).to(dev)
    w13q = torch.empty((w.E, 2 * w.I, w.H // 2), dtype=torch.uint8, device=dev)
    w13sf = torch.empty((w.E, 2 * w.I, w.H // 32), dtype=torch.uint8, device=dev)
    w2q = torch.empty((w.E, w.H, w.I // 2), dtype=torch.uint8, device=dev)
    w2sf = torch.empty((w.E, w.H, w.I // 32), dtype=torch.uint8, device=dev)

    def gen(e):
        return W.gen_expert_w13(w, e), W.gen_expert_w2(w, e)

    def up(b):
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)

    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        for e, (b13, b2) in enumerate(ex.map(gen, range(w.E))):
            w13q[e], w13sf[e] = m.pack_weights(up(b13))
            w2q[e], w2sf[e] = m.pack_weights(up(b2))
    w13sf, w2sf = m.scales_kmajor(w13sf, w.H), m.scales_kmajor(w2sf, w.I)
    torch.cuda.synchronize()
    return x, logits, w13q, w13sf, w2q, w2sf


def cpu_baseline(w, ntok):
    """The oracle on the first ntok tokens of the workload (routing of all T tokens
    included); weight quantisation is input preparation and not timed."""
    import moe_workloads as W
    from oracle import moe_ref as M

    x = W.gen_x(w)
    logits = W.gen_logits(w)
    w13, w2 = W.gen_weights(w)
    q13, s13 = M.pack_weights(w13)
    q2, s2 = M.pack_weights(w2)
    del w13, w2
    toks = np.arange(min(ntok, w.T))
    t0 = time.perf_counter()
    M.forward(x, q13, s13, q2, s2, topk=w.topk, I=w.I, logits=logits, score_fn=w.score_fn,
              renorm=bool(w.renorm), tokens=toks)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {len(toks)} of {w.T} tokens (routing, bucketisation and "
                      f"quantisation over all {w.T}); {dt:.1f} s; numpy float64 BLAS on "
                      f"{cores} host threads"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              "(the layer runs on one MI355X, see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_workloads as W
    import mixture_experts_layer_topk_amd as m

    w = W.WORKLOADS[a.workload]
    x, logits, w13q, w13sf, w2q, w2sf = setup_device(w, m, torch)
    d = m.dims(w.T, w.H, w.I, w.E, w.topk, w.score_fn, w.renorm)
    ws = m.new_workspace(d)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    flush = torch.empty(a.flush_mb << 20, dtype=torch.uint8, device="cuda") if a.flush_mb else None

    hip = Hip()
    nstage = m.NUM_STAGE_EVENTS
    ev = [(ctypes.c_void_p * nstage)(*[hip.event() for _ in range(nstage)]) for _ in range(a.steps)]
    args_plain = m.forward_args(d, x, w13q, w13sf, w2q, w2sf, y, ws, logits=logits)
    args_ev = [m.forward_args(d, x, w13q, w13sf, w2q, w2sf, y, ws, logits=logits, stage_events=e)
               for e in ev]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    if a.calib_copy_mb:
        src = torch.ones(a.calib_copy_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(a.warmup):
        m.forward_raw(args_plain, stream)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(a.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        m.forward_raw(args_ev[i], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = np.zeros(nstage - 1)
    step_ms = []
    for e in ev:
        for s in range(nstage - 1):
            stage_ms[s] += hip.elapsed_ms(e[s], e[s + 1])
        step_ms.append(hip.elapsed_ms(e[0], e[nstage - 1]))
    stage_ms /= a.steps
    ms = float(np.mean(step_ms)) if flush is not None else wall * 1e3 / a.steps
    tokens_s = w.T / (ms * 1e-3)

    R = w.T * w.topk
    gemm1_flops = 4.0 * R * w.I * w.H
    g1_tflops = gemm1_flops / (stage_ms[1] * 1e-3) / 1e12
    layer_tflops = w.flops() / (ms * 1e-3) / 1e12
    out = {
        "metric": "MoE-layer tokens/s (FP8xFP4) at DSV3 shape; % scaled-MFMA peak / HBM GB/s",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (ue8m0/32) -> fp32 acc -> bf16",
        "data": "synthetic (seeded N(0,1) x and logits, N(0,0.02) BF16 weights quantised on the GPU)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "topk": w.topk,
                   "score_fn": "sigmoid" if w.score_fn else "softmax", "renorm": bool(w.renorm),
                   "zipf_s": w.zipf_s, "parallelism": "single GPU"},
        "layer_tflops": round(layer_tflops, 2),
        "layer_frac_mfma": round(layer_tflops / PEAK_MFMA_FP8_TFLOPS, 4),
        "stages_ms": {n: round(float(v), 4) for n, v in zip(m.STAGES, stage_ms)},
        "roofline": {"kernel": "grouped_gemm_kernel<GEMM1> (FP8xFP4 MFMA + SwiGLU*w -> FP8)",
                     "bound": "mfma", "achieved": round(g1_tflops, 2),
                     "peak": PEAK_MFMA_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g1_tflops / PEAK_MFMA_FP8_TFLOPS, 4), "traffic": None},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
