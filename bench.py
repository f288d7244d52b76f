"""Benchmark of the fused FP8 x FP4 top-k MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one moe_forward call (route -> bucketise -> quantise -> GEMM1 +
SwiGLU*w -> GEMM2 -> combine) on inputs already resident in HBM.  The default
workload is the DeepSeek-V3-like one-GPU expert share (T=4096, H=7168,
I=2048, E=32, top-8).  Prints one JSON line.

The timed steps hold no events between the forward's launches.  Roofline:
per-stage times come from HIP events the library records on the launch stream
at stage boundaries, in a second pass of the same steps right after the timed
one (each such event adds about 3 us of stream time).  GEMM1 (two thirds of
the FLOPs) is reported against the dense FP8-rate MFMA peak, or, for the decode
workload, its algorithmic bytes against HBM bandwidth.  traffic is the HBM
bytes per GEMM1 launch from the committed rocprofv3 counter summary, null when
the kernel source has changed since the counters were taken.  cpu_baseline: the
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

METRIC = "MoE-layer tokens/s (FP8\u00d7FP4) at DSV3 shape; % scaled-MFMA peak / HBM GB/s"
PEAK_MFMA_FP8_TFLOPS = 5000.0      # MI355X dense FP8-rate MFMA (FP8 x FP4 issues at this rate)
PEAK_HBM_GBS = 8000.0
# workloads whose GEMMs stream more weight bytes than they have FLOPs to hide
HBM_BOUND = {"decode"}
KERNEL_SOURCES = ("gemm.hip", "narrow.hip", "narrow_dev.h", "mfma.h", "common.h", "kernels.h", "sched.h")
NARROW_ROWS_PER_EXPERT = 3         # moe_forward's choice between the two GEMM kernel families


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--tokens", type=int, default=None,
                    help="run the workload's shapes with this many tokens instead (sweeps)")
    ap.add_argument("--cpu-sample-experts", type=int, default=24,
                    help="experts whose rows the CPU oracle baseline computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weights", choices=("fp4", "fp8-block128"), default="fp4",
                    help="weight format: FP4 E2M1 + UE8M0/32 (the layer's), or the block-FP8 "
                         "variant (E4M3, one float32 scale per 128 x 128 block; narrow GEMMs)")
    ap.add_argument("--layout", choices=("staged", "canonical"), default="staged",
                    help="FP4 weight-code layout moe_forward reads: staged (moe_stage_weights, "
                         "one contiguous KiB per load) or canonical row-major")
    ap.add_argument("--gemm-path", choices=("auto", "narrow", "narrow-one-launch", "tiled", "one-launch",
                                            "one-kernel"),
                    default="auto", help="GEMM kernels moe_forward uses (default: its own choice)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before the timed steps, copy a buffer of this many MiB once (a "
                         "plain copy kernel of known size, to calibrate traffic counters)")
    ap.add_argument("--flush-mb", type=int, default=None,
                    help="read this many MiB between steps (outside the timed events) to "
                         "evict the 256 MB last-level cache; 0 = off; default 1024 for "
                         "weight-streaming (decode) workloads, whose touched experts would "
                         "otherwise stay cached, else 0.  A read leaves the cache clean, as "
                         "the weight-reading kernels between two layers would; a write would "
                         "leave it full of dirty lines whose write-backs slow the next reads")
    return ap.parse_args()


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000      # hipEventDisableSystemFence


class Hip:
    """The few HIP runtime calls the timing needs (events on the launch stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        # timing-only events: no system-scope fence (cache write-back and
        # invalidate) when recorded, which would add several us to each stage
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def setup_device(w, m, torch, fmt="fp4", layout="staged"):
    import moe_workloads as W
    from concurrent.futures import ThreadPoolExecutor

    dev = "cuda"
    x = torch.from_numpy(W.gen_x(w).view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(W.gen_logits(w)).to(dev)
    fp8 = fmt == "fp8-block128"
    if fp8:
        w13q = torch.empty((w.E, 2 * w.I, w.H), dtype=torch.uint8, device=dev)
        w13sf = torch.empty((w.E, 2 * w.I // 128, w.H // 128), dtype=torch.float32, device=dev)
        w2q = torch.empty((w.E, w.H, w.I), dtype=torch.uint8, device=dev)
        w2sf = torch.empty((w.E, w.H // 128, w.I // 128), dtype=torch.float32, device=dev)
    else:
        w13q = torch.empty((w.E, 2 * w.I, w.H // 2), dtype=torch.uint8, device=dev)
        w13sf = torch.empty((w.E, 2 * w.I, w.H // 32), dtype=torch.uint8, device=dev)
        w2q = torch.empty((w.E, w.H, w.I // 2), dtype=torch.uint8, device=dev)
        w2sf = torch.empty((w.E, w.H, w.I // 32), dtype=torch.uint8, device=dev)
    pack = m.pack_weights_fp8_block128 if fp8 else m.pack_weights

    def gen(e):
        return W.gen_expert_w13(w, e), W.gen_expert_w2(w, e)

    def up(b):
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)

    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        for e, (b13, b2) in enumerate(ex.map(gen, range(w.E))):
            w13q[e], w13sf[e] = pack(up(b13))
            w2q[e], w2sf[e] = pack(up(b2))
    if not fp8:
        w13sf, w2sf = m.scales_kmajor(w13sf, w.H), m.scales_kmajor(w2sf, w.I)
        if layout == "staged":
            w13q, w2q = m.stage_weights(w13q, True), m.stage_weights(w2q, False)
    torch.cuda.synchronize()
    return x, logits, w13q, w13sf, w2q, w2sf


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_topk_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(workload: str):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload, or None when there is none or the kernel source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm1_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def gemm1_algorithmic_bytes(w, counts, fmt="fp4") -> float:
    """Bytes GEMM1 must move at least: W1|W3 codes and scales of every expert that
    receives a row, the quantised activations once, and the h it writes (quantised;
    float32 for block-FP8 weights, quantised per 128 by the next launch)."""
    touched = int((counts > 0).sum())
    R = w.T * w.topk
    if fmt == "fp8-block128":
        w13 = 2 * w.I * w.H + (2 * w.I // 128) * (w.H // 128) * 4
        return touched * w13 + w.T * (w.H + w.H // 32) + R * w.I * 4
    w13 = 2 * w.I * (w.H // 2 + w.H // 32)
    return touched * w13 + w.T * (w.H + w.H // 32) + R * (w.I + w.I // 32)


def gemm1_kernel_name(w, path, fmt="fp4") -> str:
    if fmt == "fp8-block128":
        return "narrow_w8_gemm_kernel<GEMM1> (weight-streaming block-FP8 MFMA + SwiGLU*w -> float32 h)"
    if path == "narrow" or (path == "auto" and w.T * w.topk <= NARROW_ROWS_PER_EXPERT * w.E):
        return "narrow_gemm_kernel<GEMM1> (weight-streaming FP8xFP4 MFMA + SwiGLU*w -> FP8)"
    return "grouped_gemm_kernel<GEMM1> (tiled FP8xFP4 MFMA + SwiGLU*w -> FP8)"


def layer_algorithmic_bytes(w, counts) -> float:
    """Bytes the whole layer must move at least: W1|W3 and W2 codes and scales of every
    expert that receives a row, x, the logits and y."""
    touched = int((counts > 0).sum())
    w13 = 2 * w.I * (w.H // 2 + w.H // 32)
    w2 = w.H * (w.I // 2 + w.I // 32)
    return touched * (w13 + w2) + w.T * (2 * w.H + 4 * w.E + 2 * w.H)


def roofline(w, counts, stage_ms, path="auto", kernel_ms=None, fmt="fp4"):
    """The dominant kernel's roofline.  Its time is kernel_ms, the mean duration
    of the GEMM1 launch from the start and end events that launch carries
    (no launch gaps, no stage events inside it); without it, the GEMM1 stage
    time."""
    gemm1_ms = float(kernel_ms) if kernel_ms is not None else float(stage_ms[1])
    r = _roofline(w, counts, gemm1_ms, stage_ms, path, fmt)
    r["kernel_us"] = round(gemm1_ms * 1e3, 2)
    return r


def _roofline(w, counts, gemm1_ms, stage_ms, path, fmt="fp4"):
    if path == "one-kernel":
        # the whole layer in one kernel: its minimum bytes over its duration
        ms = float(sum(stage_ms))
        alg_bytes = layer_algorithmic_bytes(w, counts)
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        return {"kernel": "layer_small_kernel (route + quantise + narrow GEMMs + combine, one launch)",
                "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "alg_bytes": alg_bytes}
    if path == "narrow-one-launch":
        # the narrow GEMM1 and GEMM2 in one kernel: both GEMMs' minimum bytes over its duration
        touched = int((counts > 0).sum())
        w2 = w.H * (w.I // 2 + w.I // 32)
        R = w.T * w.topk
        alg_bytes = gemm1_algorithmic_bytes(w, counts) + touched * w2 + R * (w.I + w.I // 32 + 2 * w.H)
        gbs = alg_bytes / (gemm1_ms * 1e-3) / 1e9
        return {"kernel": "narrow_fused_kernel (narrow GEMM1 + SwiGLU*w + GEMM2, one launch)",
                "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "alg_bytes": alg_bytes}
    if path == "one-launch":
        # GEMM1 and GEMM2 in one kernel: all the layer's GEMM FLOPs over its duration
        tflops = w.flops() / (gemm1_ms * 1e-3) / 1e12
        return {"kernel": "fused_gemm_kernel (GEMM1 + SwiGLU*w + GEMM2, one launch)",
                "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_FP8_TFLOPS, 4),
                "traffic": None, "alg_bytes": None}
    kernel = gemm1_kernel_name(w, path, fmt)
    traffic = read_traffic(w.name) if fmt == "fp4" else None
    alg_bytes = gemm1_algorithmic_bytes(w, counts, fmt)
    if w.name in HBM_BOUND or fmt == "fp8-block128":
        gbs = alg_bytes / (gemm1_ms * 1e-3) / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic, "alg_bytes": alg_bytes}
    tflops = 4.0 * w.T * w.topk * w.I * w.H / (gemm1_ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(tflops, 2),
            "peak": PEAK_MFMA_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_FP8_TFLOPS, 4), "traffic": traffic,
            "alg_bytes": alg_bytes}


def hbm_ceiling(m, torch, hip, stream, nbytes: int, flush, steps: int):
    """The HBM read ceiling of a footprint: moe_stream_read of nbytes from a buffer
    no one has touched since the cache-evicting read, timed by the events its launch
    carries, mean over ``steps`` (the same eviction as the timed steps before each)."""
    nbytes = max(16, nbytes // 16 * 16)
    probe = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            flush.max()
        m.stream_read(probe, sink, stream, evs[i][0], evs[i][1])
    torch.cuda.synchronize()
    us = float(np.mean([hip.elapsed_ms(a, b) for a, b in evs])) * 1e3
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "stream_read_kernel (16-byte loads, nothing else)", "bytes": nbytes,
            "kernel_us": round(us, 2), "achieved": round(gbs, 1), "unit": "GB/s",
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def cpu_baseline(w, sample_experts: int, fmt: str = "fp4"):
    """The oracle, timed on a bounded sample of the workload and scaled to tokens/s.

    Timed in full: routing, bucketisation and activation quantisation of all T
    tokens, and the combine of all T tokens.  Sampled: GEMM1 -> epilogue -> GEMM2
    (the oracle's per-expert step) for every row of the first ``sample_experts``
    experts that receive rows; its time is scaled by R / (rows sampled).  Only
    the sampled experts' weights are generated and quantised (input preparation,
    not timed)."""
    import moe_workloads as W
    from oracle import blockfp8 as B
    from oracle import moe_ref as M

    fp8 = fmt == "fp8-block128"
    quant_act = B.quant_act if fp8 else M.quant_act
    pack = B.quant_weights if fp8 else M.pack_weights
    expert_rows = B.expert_rows if fp8 else M.expert_rows

    x = W.gen_x(w)
    logits = W.gen_logits(w)
    t0 = time.perf_counter()
    idx, wts = M.route(logits, w.topk, w.score_fn, bool(w.renorm))
    counts, offsets, slot_src, slot_of = M.bucketize(idx, w.E)
    xq, xsf = quant_act(x)
    t_front = time.perf_counter() - t0

    experts = [e for e in range(w.E) if counts[e] > 0][:sample_experts]
    rows = 0
    t_rows = 0.0
    o = np.zeros((int(offsets[w.E]), w.H), np.uint16)
    for e in experts:
        q13, s13 = pack(W.gen_expert_w13(w, e))
        q2, s2 = pack(W.gen_expert_w2(w, e))
        pos = np.arange(offsets[e], offsets[e + 1])
        f = slot_src[pos]
        t, j = f // w.topk, f % w.topk
        t0 = time.perf_counter()
        _, _, _, o[pos] = expert_rows(xq[t], xsf[t], wts[t, j], q13, s13, q2, s2, w.I)
        t_rows += time.perf_counter() - t0
        rows += len(pos)
    t0 = time.perf_counter()
    M.combine(o, slot_of)
    t_combine = time.perf_counter() - t0

    R = int(offsets[w.E])
    total = t_front + t_rows * R / rows + t_combine
    cores = len(os.sched_getaffinity(0))
    return {"value": w.T / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"route+bucketise+quantise of all {w.T} tokens ({t_front:.1f} s) and "
                      f"combine of all tokens ({t_combine:.1f} s) timed in full; the per-expert "
                      f"GEMM1/epilogue/GEMM2 step timed on all {rows} rows of expert(s) "
                      f"{experts} ({t_rows:.1f} s) and scaled by {R}/{rows} rows; numpy "
                      f"float64 BLAS on {cores} host threads"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              "(the layer runs on one MI355X; no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_workloads as W
    import mixture_experts_layer_topk_amd as m

    w = W.WORKLOADS[a.workload]
    if a.tokens is not None:
        from dataclasses import replace
        w = replace(w.with_tokens(a.tokens), name=f"{w.name}_T{a.tokens}")
    if a.flush_mb is None:
        a.flush_mb = 1024 if w.name in HBM_BOUND else 0
    if a.weights != "fp4":
        a.layout = "canonical"
    x, logits, w13q, w13sf, w2q, w2sf = setup_device(w, m, torch, a.weights, a.layout)
    d = m.dims(w.T, w.H, w.I, w.E, w.topk, w.score_fn, w.renorm)
    ws = m.new_workspace(d)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    flush = torch.ones(a.flush_mb << 18, dtype=torch.int32, device="cuda") if a.flush_mb else None

    hip = Hip()
    nstage = m.NUM_STAGE_EVENTS
    ev = [(ctypes.c_void_p * nstage)(*[hip.event() for _ in range(nstage)]) for _ in range(a.steps)]
    # the GEMM1 launch carries these two (its kernel's start and end times);
    # the one-kernel layer has no separate GEMM1 launch
    kev = ([(ctypes.c_void_p * 2)(hip.event(), hip.event()) for _ in range(a.steps)]
           if a.gemm_path != "one-kernel" else None)
    flags = {"auto": m.FLAG_NONE, "narrow": m.FLAG_NARROW, "tiled": m.FLAG_TILED,
             "one-launch": m.FLAG_ONE_LAUNCH, "one-kernel": m.FLAG_ONE_KERNEL,
             "narrow-one-launch": m.FLAG_NARROW | m.FLAG_ONE_LAUNCH}[a.gemm_path]
    if a.weights == "fp8-block128":
        flags |= m.FLAG_WEIGHTS_FP8_BLOCK128
    if a.layout == "staged":
        flags |= m.FLAG_W_STAGED
    args_plain = m.forward_args(d, x, w13q, w13sf, w2q, w2sf, y, ws, logits=logits, flags=flags)
    args_ev = [m.forward_args(d, x, w13q, w13sf, w2q, w2sf, y, ws, logits=logits, flags=flags,
                              stage_events=e, kernel_events=kev[i] if kev else None)
               for i, e in enumerate(ev)]
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

    # Timed steps: the forward alone, with no events between its launches (each
    # one costs about 3 us of stream time).  With the cache flush between steps
    # each step is bracketed by its own pair of events outside the forward.
    outer = [(hip.event(), hip.event()) for _ in range(a.steps)] if flush is not None else None
    t0 = time.perf_counter()
    for i in range(a.steps):
        if flush is not None:
            flush.max()
            hip.record(outer[i][0], stream)
        m.forward_raw(args_plain, stream)
        if flush is not None:
            hip.record(outer[i][1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if flush is not None:
        ms = float(np.mean([hip.elapsed_ms(b, e) for b, e in outer]))
    else:
        ms = wall * 1e3 / a.steps

    # Stage pass: the same steps again with the library's stage events, for the
    # per-stage times and the dominant kernel's duration.
    for i in range(a.steps):
        if flush is not None:
            flush.max()
        m.forward_raw(args_ev[i], stream)
    torch.cuda.synchronize()
    stage_ms = np.zeros(nstage - 1)
    for e in ev:
        for s in range(nstage - 1):
            stage_ms[s] += hip.elapsed_ms(e[s], e[s + 1])
    stage_ms /= a.steps
    # spread of the step time over the stage pass (its events add a few us per step)
    step_ms = np.array([hip.elapsed_ms(e[0], e[nstage - 1]) for e in ev])
    # the GEMM1 kernel's own duration, from the events its launch carries
    kernel_ms = float(np.mean([hip.elapsed_ms(k[0], k[1]) for k in kev])) if kev else None
    tokens_s = w.T / (ms * 1e-3)

    counts = m.intermediates(d, ws)["counts"].cpu().numpy()
    layer_tflops = w.flops() / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3 x fp4e2m1 (ue8m0/32 scales), f32 accumulate" if a.weights == "fp4" else
                  "fp8e4m3 x fp8e4m3 (f32 scales per 128x128 weight block and per 1x128 activations), "
                  "f32 accumulate"),
        "data": "synthetic (seeded N(0,1) x and logits, N(0,0.02) BF16 weights quantised on the GPU)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "topk": w.topk,
                   "score_fn": "sigmoid" if w.score_fn else "softmax", "renorm": bool(w.renorm),
                   "zipf_s": w.zipf_s, "weights": a.weights, "weight_layout": a.layout,
                   "parallelism": "single GPU"},
        "layer_tflops": round(layer_tflops, 2),
        "layer_frac_mfma": round(layer_tflops / PEAK_MFMA_FP8_TFLOPS, 4),
        "stages_ms": {n: round(float(v), 4) for n, v in zip(m.STAGES, stage_ms)},
        "stage_pass_step_ms": {q: round(float(np.percentile(step_ms, pq)), 4)
                               for q, pq in (("p10", 10), ("p50", 50), ("p90", 90))},
        "roofline": roofline(w, counts, stage_ms, a.gemm_path, kernel_ms, a.weights),
    }
    out["us_per_step"] = round(ms * 1e3, 2)
    if out["roofline"]["bound"] == "hbm":
        # the same footprint read with nothing else to do: the ceiling beside the peak
        ceil = hbm_ceiling(m, torch, hip, stream, int(out["roofline"]["alg_bytes"]), flush, a.steps)
        out["roofline"]["ceiling"] = ceil
        out["roofline"]["frac_of_ceiling"] = round(out["roofline"]["achieved"] / ceil["achieved"], 4)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_sample_experts, a.weights)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
