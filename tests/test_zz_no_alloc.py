"""moe_route_noalloc (routing with the library's static scratch instead of a
workspace) against moe_route on the same logits, through the C ABI, on two
calls in a row with the second smaller, and against the oracle.  Integer
results are bit-exact; the order inside an expert's segment is free, so
segments are compared as multisets and slot_of as their inverse."""
import sys

import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as M
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

# the largest call the scratch takes (262144 pairs, multi-workgroup routing),
# then a mid-size one, then a small one (one-workgroup routing) on the same scratch
SEQUENCE = [W.Workload("noalloc_max", T=32768, H=128, I=128, E=1024, topk=8),
            W.Workload("noalloc_mid", T=4096, H=128, I=128, E=32, topk=8, seed=1),
            W.Workload("noalloc_small", T=20, H=128, I=128, E=256, topk=8, score_fn=W.SIGMOID, seed=2)]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_route_noalloc_matches_route_on_calls_in_a_row():
    m = G.lib()
    for w in SEQUENCE:
        _log(f"route_noalloc {w.name}: T={w.T} E={w.E} k={w.topk}")
        d = m.dims(w.T, w.H, w.I, w.E, w.topk, w.score_fn, w.renorm)
        logits = G.to_dev(W.gen_logits(w))
        got = _np(m.route_noalloc(d, logits))
        torch.cuda.synchronize()
        ws = m.new_workspace(d)
        ref_gpu = _np(m.route(d, logits, ws))
        torch.cuda.synchronize()
        idx, wt = M.route(W.gen_logits(w), w.topk, w.score_fn, bool(w.renorm))
        for name in ("topk_idx", "topk_w", "counts", "offsets"):
            assert np.array_equal(got[name], ref_gpu[name]), name
        assert np.array_equal(got["topk_idx"], idx)
        np.testing.assert_allclose(got["topk_w"], wt, rtol=4e-6, atol=1e-7)
        G.check_bucketize(got, idx, w.E)
        G.check_bucketize(ref_gpu, idx, w.E)
        # a second call on the same scratch gives the same counts (its counters were cleared)
        again = _np(m.route_noalloc(d, logits))
        torch.cuda.synchronize()
        assert np.array_equal(again["counts"], got["counts"])
        del ws


def test_route_noalloc_rejects_too_many_pairs():
    m = G.lib()
    d = m.dims(32769, 128, 128, 64, 8)
    logits = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(m.MoeError) as e:
        m.route_noalloc(d, logits)       # rejected on the host before any buffer is touched
    assert e.value.code == m.MOE_ESCRATCH
