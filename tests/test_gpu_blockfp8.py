"""GPU parity of the block-FP8 (128 x 128) weight variant against its oracle
(oracle/blockfp8.py), through the C ABI: the weight packer and the activation
quantisation bit-exact (codes and float32 scales), h within the hq rule of
tests/gpu_common.py (grid steps at the larger of the two float32 scales), y within
the layer's tolerance."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import blockfp8 as B
from oracle import codecs as C
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("rows,cols", [(256, 256), (1024, 2048), (4096, 7168)])
def test_pack_weights_fp8_block128_bit_exact(rows, cols):
    _log(f"pack_weights_fp8_block128 {rows}x{cols}")
    w = W.Workload("p8", T=1, H=cols, I=rows // 2, E=1, topk=1)
    wb = W.gen_expert_w13(w, 0)[:rows]
    q, sf = G.lib().pack_weights_fp8_block128(G.bf16_dev(wb))
    torch.cuda.synchronize()
    rq, rsf = B.quant_weights(wb)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sf.cpu().numpy(), rsf)


class LayerW8:
    """A workload's inputs with block-FP8 weights packed by the library."""

    def __init__(self, w):
        m = G.lib()
        self.w = w
        self.x_np, self.logits_np = W.gen_x(w), W.gen_logits(w)
        self.x, self.logits = G.bf16_dev(self.x_np), G.to_dev(self.logits_np)
        self.w13q = torch.empty((w.E, 2 * w.I, w.H), dtype=torch.uint8, device="cuda")
        self.w13sf = torch.empty((w.E, 2 * w.I // 128, w.H // 128), dtype=torch.float32, device="cuda")
        self.w2q = torch.empty((w.E, w.H, w.I), dtype=torch.uint8, device="cuda")
        self.w2sf = torch.empty((w.E, w.H // 128, w.I // 128), dtype=torch.float32, device="cuda")
        gen = lambda e: (W.gen_expert_w13(w, e), W.gen_expert_w2(w, e))
        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            bf = list(ex.map(gen, range(w.E)))
        for e, (b13, b2) in enumerate(bf):
            self.w13q[e], self.w13sf[e] = m.pack_weights_fp8_block128(G.bf16_dev(b13))
            self.w2q[e], self.w2sf[e] = m.pack_weights_fp8_block128(G.bf16_dev(b2))
        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            self.ref_w = list(ex.map(lambda t: (*B.quant_weights(t[0]), *B.quant_weights(t[1])), bf))
        self.d = m.dims(w.T, w.H, w.I, w.E, w.topk, w.score_fn, w.renorm)
        self.ws = m.new_workspace(self.d)

    def forward(self, flags=0):
        m = G.lib()
        y = m.forward(self.d, self.x, self.w13q, self.w13sf, self.w2q, self.w2sf, self.ws,
                      logits=self.logits, flags=m.FLAG_WEIGHTS_FP8_BLOCK128 | flags)
        torch.cuda.synchronize()
        return y

    def oracle(self):
        w = self.w
        wq = [[r[i] for r in self.ref_w] for i in range(4)]
        return B.forward(self.x_np, *wq, topk=w.topk, I=w.I, logits=self.logits_np,
                         score_fn=w.score_fn, renorm=bool(w.renorm), workers=16)


def _hq_bound(ref, pairs, layer, I):
    """Accumulation-order bound of h (the same derivation as make_hq_bound) from the
    oracle's dequantised block-FP8 operands."""
    u32 = 2.0 ** -24

    def bound(rows, cols):
        out = np.empty(len(rows))
        for n, (i, c) in enumerate(zip(rows, cols)):
            f = int(pairs[i])
            t, j = f // layer.w.topk, f % layer.w.topk
            e = int(ref["topk_idx"][t, j])
            wt = float(ref["topk_w"][t, j])
            a = B.dequant_rows(ref["xq"][t], ref["xsf"][t])
            q13, s13 = layer.ref_w[e][0], layer.ref_w[e][1]
            rows13 = B.dequant_weights(q13, s13)[[c, I + c]]
            K = a.size
            g, u = float(a @ rows13[0]), float(a @ rows13[1])
            # each block's BF16 partial, then its scaling by two float32 factors
            gamma = G.accumulation_rel(K, G.MFMA_BF16_REL + 2 * u32)
            dg = gamma * float(np.abs(a) @ np.abs(rows13[0]))
            du = gamma * float(np.abs(a) @ np.abs(rows13[1]))
            silu = g / (1.0 + np.exp(-g)) if g > -700 else 0.0
            out[n] = abs(wt) * (1.1 * dg * (abs(u) + du) + (abs(silu) + 1.1 * dg) * du) + 16 * u32 * abs(silu * u * wt)
        return out

    return bound


SHAPES = [W.WORKLOADS["decode"],
          W.Workload("ragged8", T=601, H=640, I=384, E=5, topk=2),
          W.Workload("mid8", T=96, H=2048, I=512, E=32, topk=8),
          W.Workload("sig8", T=37, H=256, I=128, E=16, topk=4, score_fn=W.SIGMOID)]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_forward_block_fp8_matches_oracle(w):
    _log(f"forward block-FP8 {w.name}")
    m = G.lib()
    layer = LayerW8(w)
    # the library's packer gives the oracle's codes and scales
    for e in (0, w.E - 1):
        assert np.array_equal(layer.w13q[e].cpu().numpy(), layer.ref_w[e][0])
        assert np.array_equal(layer.w13sf[e].cpu().numpy(), layer.ref_w[e][1])
        assert np.array_equal(layer.w2q[e].cpu().numpy(), layer.ref_w[e][2])
        assert np.array_equal(layer.w2sf[e].cpu().numpy(), layer.ref_w[e][3])
    ref = layer.oracle()
    for rep in range(2):                              # the workspace is reusable
        y = layer.forward(m.FLAG_KEEP_INTERMEDIATES if rep else 0)
        inter = {k: v.cpu().numpy() for k, v in m.intermediates(layer.d, layer.ws, block_fp8=True).items()}
        assert np.array_equal(inter["topk_idx"], ref["topk_idx"])
        G.check_bucketize(inter, ref["topk_idx"], w.E)
        assert np.array_equal(inter["xq"], ref["xq"])
        assert np.array_equal(inter["xsf"], ref["xsf"])
        so_g, so_r = inter["slot_of"].reshape(-1), ref["slot_of"].reshape(-1)
        pairs = np.arange(w.T * w.topk)
        G.check_hq(inter["hq"][so_g], inter["hsf"][so_g], ref["hq"][so_r], ref["hsf"][so_r],
                   bound=_hq_bound(ref, pairs, layer, w.I), label=f"{w.name} block-FP8 hq", block=128)
        G.check_y(G.y_bits(y), ref["y"], label=f"{w.name} block-FP8 y")
