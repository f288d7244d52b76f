"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

Integer outputs (routing ids, counts, offsets, slot multisets, FP8/FP4 codes
and scales from the quantisers) must be bit-exact; floating-point outputs meet
the tolerances stated in tests/gpu_common.py.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import codecs as C
from oracle import moe_ref as M
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

# several m-tiles per expert with ragged tails, a partial GEMM2 n-tile (H % 256 != 0),
# three GEMM1 n-tiles, T not a multiple of the routing chunk
RAGGED = W.Workload("ragged", T=601, H=640, I=384, E=5, topk=2)
SMALL_SHAPES = [W.WORKLOADS["tiny"], RAGGED,
                W.Workload("k1", T=77, H=256, I=128, E=3, topk=1),
                W.Workload("sig", T=130, H=384, I=256, E=16, topk=4, score_fn=W.SIGMOID),
                W.Workload("t1", T=1, H=128, I=128, E=4, topk=2),
                # raw sigmoid weights (no renormalisation) reach the GEMM1 epilogue
                W.Workload("sig_raw", T=70, H=256, I=128, E=12, topk=3, score_fn=W.SIGMOID, renorm=0)]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_full(w, topk=None):
    x = W.gen_x(w)
    wq = G.oracle_weights(w)
    if topk is None:
        return M.forward(x, *wq, topk=w.topk, I=w.I, logits=W.gen_logits(w),
                         score_fn=w.score_fn, renorm=bool(w.renorm))
    return M.forward(x, *wq, topk=w.topk, I=w.I, topk_idx=topk[0], topk_w=topk[1])


# ------------------------------------------------------------------ quantisers

@pytest.mark.parametrize("rows,cols", [(64, 256), (5, 2048), (333, 7168)])
def test_quant_act_bit_exact(rows, cols):
    _log(f"quant_act {rows}x{cols}")
    w = W.Workload("q", T=rows, H=cols, I=128, E=1, topk=1)
    x = W.gen_x(w)
    q, sf = G.lib().quant_act(G.bf16_dev(x))
    torch.cuda.synchronize()
    rq, rsf = M.quant_act(x)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sf.cpu().numpy(), rsf)


def test_quant_act_special_values():
    _log("quant_act special values")
    vals = np.zeros((4, 64), np.float32)
    vals[1, :32] = np.array([448.0, -464.0, 2.0 ** -10, -(2.0 ** -9)] * 8)    # clamp / ties / subnormal
    vals[2, :] = -0.0
    vals[3, :] = np.ldexp(1.0, np.arange(64) % 40 - 20) * (1.75 + 2.0 ** -7)
    x = W.to_bf16_bits(vals)
    q, sf = G.lib().quant_act(G.bf16_dev(x))
    torch.cuda.synchronize()
    rq, rsf = M.quant_act(x)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sf.cpu().numpy(), rsf)


@pytest.mark.parametrize("rows,cols", [(256, 256), (1024, 2048), (4096, 7168)])
def test_pack_weights_bit_exact(rows, cols):
    _log(f"pack_weights {rows}x{cols}")
    w = W.Workload("p", T=1, H=cols, I=rows // 2, E=1, topk=1)
    wb = W.gen_expert_w13(w, 0)[:rows]
    q, sf = G.lib().pack_weights(G.bf16_dev(wb))
    torch.cuda.synchronize()
    rq, rsf = M.pack_weights(wb)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sf.cpu().numpy(), rsf)


# ------------------------------------------------------------------ routing

# 32 tokens is the most the one-workgroup routing launch takes; 33 take the
# multi-workgroup path with global counters (as do 128 and 129, with 1024 and 1032 pairs)
ROUTE_EDGES = {"tokens32": W.Workload("tokens32", T=32, H=256, I=128, E=300, topk=16),
               "tokens33": W.Workload("tokens33", T=33, H=256, I=128, E=300, topk=16),
               "pairs1024": W.Workload("pairs1024", T=128, H=256, I=128, E=32, topk=8),
               "pairs1032": W.Workload("pairs1032", T=129, H=256, I=128, E=32, topk=8),
               "e1024": W.Workload("e1024", T=3, H=128, I=128, E=1024, topk=16, score_fn=W.SIGMOID),
               # weights without renormalisation: the full softmax over E, or the raw sigmoid
               "softmax_full": W.Workload("softmax_full", T=50, H=128, I=128, E=100, topk=6, renorm=0),
               "sigmoid_raw": W.Workload("sigmoid_raw", T=40, H=128, I=128, E=200, topk=8,
                                         score_fn=W.SIGMOID, renorm=0),
               # every expert chosen by every token; many tokens on the multi-workgroup path
               "k_eq_e": W.Workload("k_eq_e", T=20, H=128, I=128, E=8, topk=8),
               "softmax_full_big": W.Workload("softmax_full_big", T=300, H=128, I=128, E=48, topk=4,
                                              renorm=0)}


@pytest.mark.parametrize("name", list(W.WORKLOADS) + list(ROUTE_EDGES))
def test_route_bit_exact(name):
    w = W.WORKLOADS.get(name) or ROUTE_EDGES[name]
    _log(f"route {name}")
    m = G.lib()
    d = m.dims(w.T, w.H, w.I, w.E, w.topk, w.score_fn, w.renorm)
    ws = m.new_workspace(d)
    logits = W.gen_logits(w)
    out = m.route(d, G.to_dev(logits), ws)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    idx, wt = M.route(logits, w.topk, w.score_fn, bool(w.renorm))
    assert np.array_equal(got["topk_idx"], idx)
    np.testing.assert_allclose(got["topk_w"], wt, rtol=4e-6, atol=1e-7)
    G.check_bucketize(got, idx, w.E)
    # the counters were reset: a second call on the same workspace gives the same counts
    out2 = m.route(d, G.to_dev(logits), ws)
    torch.cuda.synchronize()
    assert np.array_equal(out2["counts"].cpu().numpy(), got["counts"])


@pytest.mark.parametrize("T,E,topk", [(40, 64, 8), (600, 256, 8), (5, 1024, 16)])
def test_route_ties_bit_exact(T, E, topk):
    """Logits with many equal values (small integers, +0 and -0): the slots follow
    decreasing logit, equal logits by increasing expert id."""
    _log(f"route ties T={T} E={E} k={topk}")
    m = G.lib()
    d = m.dims(T, 128, 128, E, topk)
    ws = m.new_workspace(d)
    rng = np.random.default_rng(11)
    logits = rng.integers(-2, 3, (T, E)).astype(np.float32)
    logits[rng.random((T, E)) < 0.3] = -0.0
    out = m.route(d, G.to_dev(logits), ws)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    idx, wt = M.route(logits, topk)
    assert np.array_equal(got["topk_idx"], idx)
    np.testing.assert_allclose(got["topk_w"], wt, rtol=4e-6, atol=1e-7)
    G.check_bucketize(got, idx, E)


# ------------------------------------------------------------------ whole layer

@pytest.mark.parametrize("w", SMALL_SHAPES, ids=lambda w: w.name)
def test_forward_matches_oracle(w):
    _log(f"forward {w.name}")
    dl = G.DeviceLayer(w)
    y = dl.forward()
    inter = dl.intermediates()
    ref = _oracle_full(w)
    assert np.array_equal(inter["topk_idx"], ref["topk_idx"])
    G.check_bucketize(inter, ref["topk_idx"], w.E)
    assert np.array_equal(inter["xq"], ref["xq"])
    assert np.array_equal(inter["xsf"], ref["xsf"])
    # hq by (t, j): map GPU positions and oracle positions through slot_of
    so_g = inter["slot_of"].reshape(-1)
    so_r = ref["slot_of"].reshape(-1)
    G.check_hq(inter["hq"][so_g], inter["hsf"][so_g], ref["hq"][so_r], ref["hsf"][so_r])
    G.check_y(G.y_bits(y), ref["y"])


def test_forward_decode_matches_oracle():
    w = W.WORKLOADS["decode"]
    _log("forward decode")
    dl = G.DeviceLayer(w)
    y = dl.forward()
    ref = _oracle_full(w)
    inter = dl.intermediates()
    so_g, so_r = inter["slot_of"].reshape(-1), ref["slot_of"].reshape(-1)
    G.check_hq(inter["hq"][so_g], inter["hsf"][so_g], ref["hq"][so_r], ref["hsf"][so_r])
    G.check_y(G.y_bits(y), ref["y"])


@pytest.mark.parametrize("name", ["dsv3_prefill", "dsv3_skewed", "full256"])
def test_forward_full_size_sampled_tokens(name):
    """Full-size launch; the oracle recomputes a sample of tokens one by one (only
    the experts those tokens touch are generated and quantised on its side)."""
    w = W.WORKLOADS[name]
    _log(f"forward {name} (sampled)")
    dl = G.DeviceLayer(w)
    y = dl.forward()
    inter = dl.intermediates()
    logits = dl.logits_np
    idx, _ = M.route(logits, w.topk, w.score_fn, bool(w.renorm))
    assert np.array_equal(inter["topk_idx"], idx)
    G.check_bucketize(inter, idx, w.E)
    toks = [0, w.T // 3, 2 * w.T // 3, w.T - 1]
    ref = M.forward(dl.x_np, *G.oracle_weights(w), topk=w.topk, I=w.I, logits=logits,
                    score_fn=w.score_fn, renorm=bool(w.renorm), tokens=toks)
    G.check_y(G.y_bits(y), ref["y"], rows=toks)
    so_g = inter["slot_of"][toks].reshape(-1)
    so_r = ref["slot_of"][toks].reshape(-1)
    G.check_hq(inter["hq"][so_g], inter["hsf"][so_g], ref["hq"][so_r], ref["hsf"][so_r])
    # every output row is finite and the untouched workspace regions stay consistent
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("path", ["narrow", "tiled"])
def test_token_permutation_permutes_y_bit_exactly(path):
    """Each output row depends only on its own token, and each accumulation runs in a
    fixed order whatever a row's position inside its expert segment, so permuting the
    tokens permutes y bit for bit (the oracle's own permutation pin, on the GPU)."""
    m = G.lib()
    _log(f"token permutation ({path})")
    flags = m.FLAG_NARROW if path == "narrow" else m.FLAG_TILED
    dl = G.DeviceLayer(RAGGED)
    y = dl.forward(flags=flags).clone()
    perm = torch.from_numpy(np.random.default_rng(3).permutation(RAGGED.T)).to(y.device)
    dl.x = dl.x[perm].contiguous()
    dl.logits = dl.logits[perm].contiguous()
    y_perm = dl.forward(flags=flags)
    assert torch.equal(y_perm.view(torch.int16), y[perm].view(torch.int16))


def test_forward_external_topk_with_masked_slots():
    w = W.Workload("ext", T=257, H=256, I=256, E=6, topk=3)
    _log("forward external topk")
    topk = W.gen_external_topk(w, mask_frac=0.25)
    dl = G.DeviceLayer(w, external_topk=topk)
    y = dl.forward(use_logits=False)
    ref = _oracle_full(w, topk)
    inter = dl.intermediates()
    G.check_bucketize(inter, topk[0], w.E)
    G.check_y(G.y_bits(y), ref["y"])


def test_forward_all_tokens_one_expert():
    w = W.Workload("hot", T=700, H=256, I=128, E=8, topk=1)
    _log("forward one hot expert")
    idx = np.full((w.T, 1), 5, np.int32)
    wt = np.ones((w.T, 1), np.float32)
    dl = G.DeviceLayer(w, external_topk=(idx, wt))
    y = dl.forward(use_logits=False)
    ref = _oracle_full(w, (idx, wt))
    G.check_y(G.y_bits(y), ref["y"])


def test_forward_is_deterministic_and_workspace_reusable():
    w = RAGGED
    _log("determinism")
    dl = G.DeviceLayer(w)
    ys = [G.y_bits(dl.forward()) for _ in range(3)]
    assert all(np.array_equal(ys[0], v) for v in ys[1:])
    # a smaller call on the same workspace, then the full call again
    m = G.lib()
    d_small = m.dims(100, w.H, w.I, w.E, w.topk)
    y_small = m.forward(d_small, dl.x[:100], dl.w13q, dl.w13sf_k, dl.w2q, dl.w2sf_k, dl.ws,
                        logits=dl.logits[:100])
    torch.cuda.synchronize()
    ref_small = M.forward(dl.x_np[:100], *G.oracle_weights(w), topk=w.topk, I=w.I,
                          logits=dl.logits_np[:100])
    G.check_y(G.y_bits(y_small), ref_small["y"])
    assert np.array_equal(G.y_bits(dl.forward()), ys[0])


# few rows per expert (decode), more than 16 rows per expert (several 16-row passes of the
# narrow kernels), K-step counts below and not a multiple of the narrow kernels' four-way
# K split, and all rows on one expert
AGREE_SHAPES = [W.WORKLOADS["decode"], W.WORKLOADS["tiny"], RAGGED,
                W.Workload("mid", T=96, H=2048, I=512, E=32, topk=8),
                W.Workload("hot1", T=300, H=256, I=128, E=8, topk=1)]


@pytest.mark.parametrize("w", AGREE_SHAPES, ids=lambda w: w.name)
def test_narrow_and_tiled_gemms_match_oracle(w):
    """Every GEMM path (narrow in two launches or one; tiled in one launch or two),
    forced on the same inputs, against the oracle (the default picks one per shape)."""
    m = G.lib()
    _log(f"narrow and tiled {w.name}")
    ext = None
    if w.name == "hot1":
        ext = (np.full((w.T, 1), 3, np.int32), np.ones((w.T, 1), np.float32))
    dl = G.DeviceLayer(w, external_topk=ext)
    ref = _oracle_full(w, ext)
    so_r = ref["slot_of"].reshape(-1)
    paths = [("narrow", m.FLAG_NARROW), ("narrow, one launch", m.FLAG_NARROW | m.FLAG_ONE_LAUNCH),
             ("tiled, two launches", m.FLAG_TILED), ("tiled, one launch", m.FLAG_ONE_LAUNCH)]
    if w.T * w.topk <= 1024:
        paths.append(("whole layer, one kernel", m.FLAG_ONE_KERNEL))
    for name, flag in paths:
        _log(f"  {name}")
        y = dl.forward(use_logits=ext is None, flags=flag)
        inter = dl.intermediates()
        so_g = inter["slot_of"].reshape(-1)
        ok = so_r >= 0
        G.check_hq(inter["hq"][so_g[ok]], inter["hsf"][so_g[ok]], ref["hq"][so_r[ok]],
                   ref["hsf"][so_r[ok]])
        G.check_y(G.y_bits(y), ref["y"])


# More tiles than workgroups, so that workgroups run several tiles back to back:
# "chain" has enough K steps in both GEMMs for the next tile to be set up inside
# the current one's K loop; "short_k" has too few (GEMM1 4 steps, GEMM2 1) and
# sets up every tile after the previous one; "chain_k2" chains GEMM2 tiles of
# the fewest K steps that allow it (2), so the next tile's set-up shares the
# step that issues its first loads.
MULTI_TILE_SHAPES = [W.Workload("chain", T=3072, H=768, I=512, E=8, topk=8),
                     W.Workload("short_k", T=4096, H=512, I=128, E=8, topk=8),
                     W.Workload("chain_k2", T=4096, H=512, I=256, E=8, topk=8)]


@pytest.mark.parametrize("w", MULTI_TILE_SHAPES, ids=lambda w: w.name)
def test_tiled_gemms_many_tiles_per_workgroup(w):
    m = G.lib()
    _log(f"many tiles per workgroup {w.name}")
    dl = G.DeviceLayer(w)
    ref = _oracle_full(w)
    so_r = ref["slot_of"].reshape(-1)
    for name, flag in (("tiled, two launches", m.FLAG_TILED),
                       ("tiled, one launch", m.FLAG_ONE_LAUNCH)):
        _log(f"  {name}")
        y = dl.forward(flags=flag)
        inter = dl.intermediates()
        so_g = inter["slot_of"].reshape(-1)
        G.check_hq(inter["hq"][so_g], inter["hsf"][so_g], ref["hq"][so_r], ref["hsf"][so_r])
        G.check_y(G.y_bits(y), ref["y"])


def test_one_launch_reads_this_calls_h():
    """Alternating two different inputs on one workspace: a GEMM2 tile that read h
    left in a cache by the previous call (instead of this call's GEMM1 tiles) would
    give the other input's result."""
    m = G.lib()
    wa, wb = RAGGED, W.Workload("ragged_b", T=601, H=640, I=384, E=5, topk=2, seed=1)
    _log("one launch, alternating inputs")
    da, db = G.DeviceLayer(wa), G.DeviceLayer(wb)
    db.ws = da.ws
    ra, rb = _oracle_full(wa), _oracle_full(wb)
    for dl, ref in ((da, ra), (db, rb), (da, ra), (db, rb)):
        y = dl.forward(flags=m.FLAG_ONE_LAUNCH)
        G.check_y(G.y_bits(y), ref["y"])


def test_narrow_one_launch_reads_this_calls_h():
    """The narrow GEMMs in one launch on alternating inputs and shapes sharing one
    workspace: a GEMM2 unit that read h left in a cache by the previous call, or
    started before this call's GEMM1 units of its sub-tile had stored theirs, would
    give the other input's result."""
    m = G.lib()
    wa = W.WORKLOADS["decode"]
    wb = W.Workload("decode_b", T=8, H=2048, I=512, E=256, topk=8, seed=1)
    wc = W.Workload("mid_b", T=96, H=2048, I=512, E=32, topk=8, seed=2)
    _log("narrow one launch, alternating inputs")
    da, db, dc = G.DeviceLayer(wa), G.DeviceLayer(wb), G.DeviceLayer(wc)
    db.ws = da.ws
    if dc.ws.numel() > da.ws.numel():
        da.ws = db.ws = dc.ws
    else:
        dc.ws = da.ws
    refs = [_oracle_full(w) for w in (wa, wb, wc)]
    for _ in range(2):
        for dl, ref in zip((da, db, dc), refs):
            y = dl.forward(flags=m.FLAG_NARROW | m.FLAG_ONE_LAUNCH)
            G.check_y(G.y_bits(y), ref["y"])


def test_one_kernel_layer_reads_this_calls_data():
    """The one-kernel layer on alternating inputs and shapes sharing one workspace: a
    phase that read a previous call's activations, tables or GEMM outputs from a stale
    cache line (instead of what this call's earlier phase stored), or a barrier counter
    left non-zero by the previous call, would give the other input's result."""
    m = G.lib()
    wa = W.WORKLOADS["decode"]
    wb = W.Workload("decode_b", T=8, H=2048, I=512, E=256, topk=8, seed=1)
    wc = W.Workload("mid_b", T=96, H=2048, I=512, E=32, topk=8, seed=2)
    _log("one kernel, alternating inputs")
    da, db, dc = G.DeviceLayer(wa), G.DeviceLayer(wb), G.DeviceLayer(wc)
    db.ws = da.ws
    if dc.ws.numel() > da.ws.numel():
        da.ws = db.ws = dc.ws
    else:
        dc.ws = da.ws
    refs = [_oracle_full(w) for w in (wa, wb, wc)]
    for _ in range(2):
        for dl, ref in zip((da, db, dc), refs):
            y = dl.forward(flags=m.FLAG_ONE_KERNEL)
            G.check_y(G.y_bits(y), ref["y"])


def test_scales_kmajor_is_a_transpose():
    _log("scales_kmajor")
    rng = np.random.default_rng(5)
    sf = rng.integers(0, 255, (3, 40, 7168 // 32), dtype=np.uint8)
    out = G.lib().scales_kmajor(G.to_dev(sf), 7168).cpu().numpy()
    assert np.array_equal(out, sf.reshape(3, 40, 7168 // 128, 4).transpose(0, 2, 1, 3))


def test_forward_zero_tokens_is_noop():
    m = G.lib()
    d = m.dims(0, 256, 128, 4, 2)
    ws = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda")
    y = torch.full((1, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(64, dtype=torch.uint8, device="cuda")
    m.forward_raw(m.forward_args(d, x, w, w, w, w, y, ws, logits=x))
    torch.cuda.synchronize()
    assert (y.float() == 7.0).all()


@pytest.mark.parametrize("flags", ["tiled", "narrow", "one-launch", "narrow-one-launch", "one-kernel"])
def test_timing_events_leave_y_unchanged(flags):
    """Stage events and the GEMM1 launch's own events change nothing in y; the
    GEMM1 kernel's start-to-end time is positive and inside its stage.  The
    one-kernel layer records its stage events and leaves the kernel pair alone."""
    m = G.lib()
    f = {"tiled": m.FLAG_TILED, "narrow": m.FLAG_NARROW, "one-launch": m.FLAG_ONE_LAUNCH,
         "narrow-one-launch": m.FLAG_NARROW | m.FLAG_ONE_LAUNCH,
         "one-kernel": m.FLAG_ONE_KERNEL}[flags]
    w = W.WORKLOADS["decode"] if flags == "one-kernel" else RAGGED
    _log(f"timing events {flags}")
    dl = G.DeviceLayer(w)
    ref = G.y_bits(dl.forward(flags=f))
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event():
        e = ctypes.c_void_p()
        assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) == 0   # no system fence
        return e

    def elapsed(a, b):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    sev = (ctypes.c_void_p * m.NUM_STAGE_EVENTS)(*[event() for _ in range(m.NUM_STAGE_EVENTS)])
    kev = (ctypes.c_void_p * 2)(event(), event())
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    args = m.forward_args(dl.d, dl.x, dl.w13q, dl.w13sf_k, dl.w2q, dl.w2sf_k, y, dl.ws,
                          logits=dl.logits, flags=f, stage_events=sev, kernel_events=kev)
    for _ in range(2):
        m.forward_raw(args)
        torch.cuda.synchronize()
        assert np.array_equal(G.y_bits(y), ref)
        stages = [elapsed(sev[i], sev[i + 1]) for i in range(m.NUM_STAGE_EVENTS - 1)]
        assert all(t >= 0.0 for t in stages) and sum(stages) > 0.0, stages
        if flags != "one-kernel":
            kernel = elapsed(kev[0], kev[1])
            assert 0.0 < kernel <= stages[1] + 1e-3, (kernel, stages)
    for e in list(sev) + list(kev):
        hip.hipEventDestroy(e)
