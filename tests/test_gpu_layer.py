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

def _pairs_of(w, tokens=None):
    if tokens is None:
        return np.arange(w.T * w.topk)
    return (np.asarray(tokens)[:, None] * w.topk + np.arange(w.topk)[None, :]).reshape(-1)


def _check_layer(inter, y, ref, w, label, tokens=None):
    """hq of every compared (token, slot) pair, matched through slot_of on each side,
    and y of every compared token, against the oracle (tolerances in gpu_common)."""
    so_g = inter["slot_of"].reshape(-1)
    so_r = ref["slot_of"].reshape(-1)
    pairs = _pairs_of(w, tokens)
    pairs = pairs[so_r[pairs] >= 0]                 # masked slots have no row
    wq = G.oracle_weights(w)
    bound = G.make_hq_bound(ref, pairs, wq[0], wq[1], w.topk, w.I)
    G.check_hq(inter["hq"][so_g[pairs]], inter["hsf"][so_g[pairs]], ref["hq"][so_r[pairs]],
               ref["hsf"][so_r[pairs]], bound=bound, label=f"{label} hq")
    G.check_y(G.y_bits(y), ref["y"], rows=tokens, label=f"{label} y")


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
    _check_layer(inter, y, ref, w, w.name)


def test_forward_decode_matches_oracle():
    w = W.WORKLOADS["decode"]
    _log("forward decode")
    dl = G.DeviceLayer(w)
    y = dl.forward()
    ref = _oracle_full(w)
    _check_layer(dl.intermediates(), y, ref, w, "decode")


# Full-size workloads: the device layer and the oracle's result are built once per
# workload and shared by the tests that use them.
_BIG = {}


def _big(name, tokens=None):
    key = (name, None if tokens is None else tuple(tokens))
    if key not in _BIG:
        w = W.WORKLOADS[name]
        dl = _BIG.get((name, "layer")) or G.DeviceLayer(w)
        _BIG[(name, "layer")] = dl
        experts = None
        if tokens is not None:
            idx, _ = M.route(dl.logits_np, w.topk, w.score_fn, bool(w.renorm))
            experts = np.unique(idx[np.asarray(tokens)])
        G.prefetch_oracle_experts(w, experts)
        _BIG[key] = M.forward(dl.x_np, *G.oracle_weights(w), topk=w.topk, I=w.I, logits=dl.logits_np,
                              score_fn=w.score_fn, renorm=bool(w.renorm), tokens=tokens, workers=16)
    return _BIG[(name, "layer")], _BIG[key]


@pytest.mark.parametrize("name", ["dsv3_prefill", "dsv3_skewed"])
def test_forward_full_size_every_token(name):
    """The DeepSeek-V3-like shapes in full, with the staged weight codes the
    benchmark runs: every token's y and every pair's hq (the whole 56-step K loop,
    every m-tile of every expert, the skewed workload's hot and near-empty experts)
    against the oracle on all tokens; then the canonical layout, bit for bit."""
    w = W.WORKLOADS[name]
    _log(f"forward {name} (every token)")
    dl, ref = _big(name)
    y = dl.forward(staged=True)
    inter = dl.intermediates()
    assert np.array_equal(inter["topk_idx"], ref["topk_idx"])
    G.check_bucketize(inter, ref["topk_idx"], w.E)
    assert np.array_equal(inter["xq"], ref["xq"])
    assert np.array_equal(inter["xsf"], ref["xsf"])
    _check_layer(inter, y, ref, w, name)
    y_c = dl.forward()
    assert np.array_equal(G.y_bits(y_c), G.y_bits(y)), "canonical and staged weight layouts differ"
    # hq row by routed pair (the order of pairs inside an expert's segment is not fixed)
    inter_c = dl.intermediates()
    so, so_c = inter["slot_of"].reshape(-1), inter_c["slot_of"].reshape(-1)
    assert np.array_equal(inter_c["hq"][so_c], inter["hq"][so])
    assert np.array_equal(inter_c["hsf"][so_c], inter["hsf"][so])


def _fused_waves(w):
    """Expert waves of the one-launch list on this GPU (the launcher's formula)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nt1 = (w.I + 255) // 256
    per_expert = max(1, -(-w.T * w.topk // w.E))
    tiles = -(-per_expert // 128) * nt1
    ew = min(w.E, max(1, -(-2 * cus // tiles)))
    return -(-w.E // ew)


def test_one_launch_full_size_dsv3_prefill():
    """The one-launch scheduler at the DeepSeek-V3-like shape (4 expert waves on
    256 CUs: GEMM1 of wave w + 1 runs between GEMM1 and GEMM2 of wave w), every
    token against the oracle."""
    m = G.lib()
    w = W.WORKLOADS["dsv3_prefill"]
    waves = _fused_waves(w)
    _log(f"one launch dsv3_prefill (every token, {waves} expert waves)")
    assert waves >= 2
    dl, ref = _big("dsv3_prefill")
    y = dl.forward(flags=m.FLAG_ONE_LAUNCH)
    _check_layer(dl.intermediates(), y, ref, w, f"one launch, {waves} waves")


def _full256_tokens(inter, w):
    """One token in the last (ragged) 128-row m-tile of every expert, by the GPU's
    own positions, plus a seeded sample of 64 tokens."""
    off = inter["offsets"]
    src = inter["slot_src"]
    toks = set()
    for e in range(w.E):
        if off[e + 1] > off[e]:
            toks.add(int(src[off[e + 1] - 1]) // w.topk)     # last row of the last m-tile
    toks |= set(np.random.default_rng(1234).choice(w.T, 64, replace=False).tolist())
    return sorted(toks)


@pytest.mark.parametrize("flags", ["default", "one-launch"])
def test_forward_full256_every_expert_tail(flags):
    """256 experts on one GPU (8 expert waves in the one-launch list): y and hq of
    tokens covering the last, ragged m-tile of every expert."""
    m = G.lib()
    w = W.WORKLOADS["full256"]
    _log(f"forward full256 ({flags}; one token in every expert's last m-tile)")
    dl = _BIG.get(("full256", "layer")) or G.DeviceLayer(w)
    _BIG[("full256", "layer")] = dl
    f = m.FLAG_ONE_LAUNCH if flags == "one-launch" else m.FLAG_NONE
    y = dl.forward(flags=f, staged=True)
    inter = dl.intermediates()
    counts = inter["counts"]
    ragged = int(((counts % 128) != 0).sum())
    if ("full256", "tokens") not in _BIG:
        _BIG[("full256", "tokens")] = _full256_tokens(inter, w)
    toks = _BIG[("full256", "tokens")]
    _log(f"  {len(toks)} tokens; {ragged} of {w.E} experts end in a partial m-tile; "
         f"{_fused_waves(w)} expert waves")
    dl2, ref = _big("full256", toks)
    assert np.array_equal(inter["topk_idx"], ref["topk_idx"])
    G.check_bucketize(inter, ref["topk_idx"], w.E)
    _check_layer(inter, y, ref, w, f"full256 {flags}", tokens=toks)
    y_c = dl.forward(flags=f)
    assert np.array_equal(G.y_bits(y_c), G.y_bits(y)), "canonical and staged weight layouts differ"


# Shapes whose one-launch list has several expert waves on 256 CUs (3072 rows per
# expert on average: 24 m-tiles x 8 GEMM1 n-tiles, so 3 experts per wave), with
# uniform and Zipf-skewed routing
WAVE_SHAPES = [W.Workload("wave_uniform", T=3072, H=256, I=2048, E=8, topk=8),
               W.Workload("wave_skewed", T=6144, H=256, I=2048, E=8, topk=4, zipf_s=1.2)]


@pytest.mark.parametrize("w", WAVE_SHAPES, ids=lambda w: w.name)
def test_one_launch_multi_wave(w):
    m = G.lib()
    waves = _fused_waves(w)
    _log(f"one launch {w.name} ({waves} expert waves)")
    assert waves >= 2, "the shape must give several expert waves"
    dl = G.DeviceLayer(w)
    ref = _oracle_full(w)
    for name, flag in (("one launch", m.FLAG_ONE_LAUNCH), ("two launches", m.FLAG_TILED)):
        y = dl.forward(flags=flag)
        inter = dl.intermediates()
        _log(f"  {name}: counts {inter['counts'].tolist()}")
        _check_layer(inter, y, ref, w, f"{w.name} {name}")


def test_workspace_poisoned_except_counters():
    """After moe_workspace_init, every workspace byte past the counter header is set
    to 0xFF: each path must write every region it reads (only the counters need the
    one-time zeroing)."""
    m = G.lib()
    w = RAGGED
    _log("poisoned workspace")
    dl = G.DeviceLayer(w)
    ref = _oracle_full(w)
    status_off = m.workspace_layout(dl.d).status
    for name, flag in (("default", m.FLAG_NONE), ("narrow", m.FLAG_NARROW), ("tiled", m.FLAG_TILED),
                       ("one launch", m.FLAG_ONE_LAUNCH), ("narrow one launch", m.FLAG_NARROW | m.FLAG_ONE_LAUNCH)):
        dl.ws[status_off:] = 0xFF
        y = dl.forward(flags=flag)
        _check_layer(dl.intermediates(), y, ref, w, f"poisoned, {name}")
    wd = W.WORKLOADS["decode"]
    dd = G.DeviceLayer(wd)
    refd = _oracle_full(wd)
    dd.ws[m.workspace_layout(dd.d).status:] = 0xFF
    y = dd.forward(flags=m.FLAG_ONE_KERNEL)
    _check_layer(dd.intermediates(), y, refd, wd, "poisoned, one kernel")


@pytest.mark.parametrize("w", [RAGGED, W.WORKLOADS["decode"]], ids=lambda w: w.name)
def test_weight_layout_flags(w):
    """Pre-interleaved W13 (the pages' gran-8 gate/up interleave, built by the
    oracle's interleave from the oracle-packed weights), per-row weight scales and
    the staged weight codes give the oracle's result on every GEMM path (the
    ragged shape has partial last n-tiles in both GEMMs), bit-identical to the
    canonical layout."""
    m = G.lib()
    _log(f"weight layout flags {w.name}")
    dl = G.DeviceLayer(w)
    ref = _oracle_full(w)
    G.prefetch_oracle_experts(w)
    q13 = np.stack([G.oracle_expert(w, e)[0] for e in range(w.E)])
    s13 = np.stack([G.oracle_expert(w, e)[1] for e in range(w.E)])
    iq, isf = M.interleave_w13(q13, s13)
    iq_d, isf_d = G.to_dev(iq), G.to_dev(isf)
    isf_k = m.scales_kmajor(isf_d, w.H)
    paths = [("narrow", m.FLAG_NARROW), ("tiled", m.FLAG_TILED), ("one launch", m.FLAG_ONE_LAUNCH),
             ("narrow one launch", m.FLAG_NARROW | m.FLAG_ONE_LAUNCH)]
    if w.T * w.topk <= 1024:
        paths.append(("one kernel", m.FLAG_ONE_KERNEL))
    for name, flag in paths:
        base = G.y_bits(dl.forward(flags=flag))
        s13, s2 = dl.staged()
        variants = {
            "interleaved": (iq_d, isf_k, dl.w2q, dl.w2sf_k, m.FLAG_W13_PREINTERLEAVED),
            "per-row scales": (dl.w13q, dl.w13sf, dl.w2q, dl.w2sf, m.FLAG_W_SCALES_PER_ROW),
            "both": (iq_d, isf_d, dl.w2q, dl.w2sf, m.FLAG_W13_PREINTERLEAVED | m.FLAG_W_SCALES_PER_ROW),
            "staged": (s13, dl.w13sf_k, s2, dl.w2sf_k, m.FLAG_W_STAGED),
            "staged, per-row scales": (s13, dl.w13sf, s2, dl.w2sf, m.FLAG_W_STAGED | m.FLAG_W_SCALES_PER_ROW),
        }
        for vname, (a13, b13, a2, b2, vf) in variants.items():
            y = m.forward(dl.d, dl.x, a13, b13, a2, b2, dl.ws, logits=dl.logits,
                          flags=flag | vf | m.FLAG_KEEP_INTERMEDIATES)
            torch.cuda.synchronize()
            _check_layer(dl.intermediates(), y, ref, w, f"{name}, {vname}")
            assert np.array_equal(G.y_bits(y), base), f"{name}, {vname}: y differs from the canonical layout"


def test_check_status_reports_the_status_word():
    """moe_check_status reads the status word a call leaves; a forward clears it."""
    m = G.lib()
    w = RAGGED
    _log("check_status")
    dl = G.DeviceLayer(w)
    dl.forward()
    assert m.check_status(dl.ws) == m.MOE_OK
    status_off = m.workspace_layout(dl.d).status
    dl.ws[status_off:status_off + 4] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
    assert m.check_status(dl.ws) == m.MOE_ETIMEOUT
    dl.forward()
    assert m.check_status(dl.ws) == m.MOE_OK


@pytest.mark.parametrize("w", [WAVE_SHAPES[0], W.WORKLOADS["decode"]], ids=lambda w: w.name)
def test_debug_spin_bound_ends_and_reports(w):
    """With DEBUG_SPIN_BOUND every ready-counter wait of the one-launch paths gives
    up after one failed poll: the call still ends, and moe_check_status agrees with
    the status word; the next call without the flag is correct again."""
    m = G.lib()
    _log(f"debug spin bound {w.name}")
    dl = G.DeviceLayer(w)
    ref = _oracle_full(w)
    base = m.FLAG_NARROW | m.FLAG_ONE_LAUNCH if w.name == "decode" else m.FLAG_ONE_LAUNCH
    for _ in range(3):
        m.forward(dl.d, dl.x, dl.w13q, dl.w13sf_k, dl.w2q, dl.w2sf_k, dl.ws, logits=dl.logits,
                  flags=base | m.FLAG_DEBUG_SPIN_BOUND)
        rc = m.check_status(dl.ws)
        word = int(m.intermediates(dl.d, dl.ws)["status"].item())
        _log(f"  status word {word}, check_status {rc}")
        assert rc == (m.MOE_OK if word == 0 else m.MOE_ETIMEOUT)
    y = dl.forward(flags=base)
    assert m.check_status(dl.ws) == m.MOE_OK
    _check_layer(dl.intermediates(), y, ref, w, f"{w.name} after debug spin bound")


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


def _combine_of(o_bits, slot_of, H):
    """y from the GPU's own GEMM2 rows, by the combine's definition: float32 sums
    in slot order (0 + row of slot 0 + row of slot 1 ...), skipped slots adding
    nothing, rounded to BF16."""
    acc = np.zeros((slot_of.shape[0], H), np.float32)
    for j in range(slot_of.shape[1]):
        pos = slot_of[:, j]
        ok = pos >= 0
        acc[ok] = acc[ok] + C.bf16_value(o_bits[pos[ok]])
    return C.bf16_bits(acc)


# The narrow path with a caller's top-k: routing through the one-workgroup
# bucketing (decode, 8 tokens) and the multi-workgroup one (40 tokens)
COMBINE_SHAPES = [W.WORKLOADS["decode"], W.Workload("narrow40", T=40, H=512, I=256, E=64, topk=4)]


@pytest.mark.parametrize("w", COMBINE_SHAPES, ids=lambda w: w.name)
def test_narrow_path_combine_is_exact(w):
    """On the narrow GEMMs, y equals the slot-order combine of the GPU's own GEMM2
    rows bit for bit, with masked slots and one token with none (y = 0), and
    matches the oracle."""
    _log(f"narrow path combine {w.name}")
    idx, wt = W.gen_external_topk(w, mask_frac=0.25)
    idx[0] = -1                                  # token 0: no expert at all
    dl = G.DeviceLayer(w, external_topk=(idx, wt))
    assert w.T * w.topk <= 3 * w.E, "the shape must take the narrow GEMMs"
    y = dl.forward(use_logits=False)
    inter = dl.intermediates()
    o = inter["o"].view(np.uint16)
    yb = G.y_bits(y)
    assert np.array_equal(yb, _combine_of(o, inter["slot_of"], w.H)), "y is not the combine of GEMM2's rows"
    assert not yb[0].any(), "a token without experts must give y = 0"
    ref = _oracle_full(w, (idx, wt))
    G.check_y(yb, ref["y"], label=f"{w.name} y")
    # a second call on the same workspace (the counters start from zero again)
    y2 = dl.forward(use_logits=False)
    assert np.array_equal(G.y_bits(y2), yb)


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
    paths = [("narrow", m.FLAG_NARROW), ("narrow, one launch", m.FLAG_NARROW | m.FLAG_ONE_LAUNCH),
             ("tiled, two launches", m.FLAG_TILED), ("tiled, one launch", m.FLAG_ONE_LAUNCH)]
    if w.T * w.topk <= 1024:
        paths.append(("whole layer, one kernel", m.FLAG_ONE_KERNEL))
    for name, flag in paths:
        _log(f"  {name}")
        y = dl.forward(use_logits=ext is None, flags=flag)
        _check_layer(dl.intermediates(), y, ref, w, f"{w.name} {name}")


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
    for name, flag in (("tiled, two launches", m.FLAG_TILED),
                       ("tiled, one launch", m.FLAG_ONE_LAUNCH)):
        _log(f"  {name}")
        y = dl.forward(flags=flag)
        _check_layer(dl.intermediates(), y, ref, w, f"{w.name} {name}")
        y_s = dl.forward(flags=flag, staged=True)
        assert np.array_equal(G.y_bits(y_s), G.y_bits(y)), f"{name}: staged weight codes change y"


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


def _staged_reference(q, is_w13):
    """The staged layout written out from its definition: rows in groups of 16,
    group g = 8 b + n holding canonical rows (n & 1) * I + 64 b + 4 c + n // 2
    (W13) or 128 b + 8 c + n (W2), c < 16; per group, K step after K step, the
    16 rows' 64 bytes of that step."""
    mats, rows, kb = q.shape
    nk = kb // 64
    g = np.arange(rows // 16)[:, None]
    c = np.arange(16)[None, :]
    if is_w13:
        row = (g & 1) * (rows // 2) + 64 * (g >> 3) + 4 * c + ((g & 7) >> 1)
    else:
        row = 128 * (g >> 3) + 8 * c + (g & 7)
    assert np.array_equal(np.sort(row.reshape(-1)), np.arange(rows)), "not a permutation of the rows"
    src = q.reshape(mats, rows, nk, 64)[:, row]               # [mats, groups, 16, nk, 64]
    return np.ascontiguousarray(src.transpose(0, 1, 3, 2, 4)).reshape(mats, rows, kb)


@pytest.mark.parametrize("mats,rows,cols,is_w13", [(3, 256, 256, True), (2, 768, 640, True),
                                                   (4, 640, 384, False), (1, 7168, 2048, False),
                                                   (2, 4096, 7168, True)])
def test_stage_weights_layout(mats, rows, cols, is_w13):
    m = G.lib()
    q = np.random.default_rng(7).integers(0, 256, (mats, rows, cols // 2), dtype=np.uint8)
    out = m.stage_weights(G.to_dev(q), is_w13).cpu().numpy()
    assert np.array_equal(out, _staged_reference(q, is_w13))


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
