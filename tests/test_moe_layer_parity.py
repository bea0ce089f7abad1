"""GPU parity of the MoE decode layer call (qmm_moe_layer): stage 1 (gathered
gate+up+SwiGLU, touching the routed experts' down rows on the way) and stage 2 (gathered
down + weighted combine) of one token in one call.

Checks: h against the fp64 oracle at the SwiGLU bound; h and y equal, bit for bit, the two
qmm_moe_gather calls on the same inputs (stage 2 of those calls reads the GPU's own h, as
the layer does; stage 2 itself is checked against the oracle on the oracle's h in
test_moe_parity.py, so no GPU value enters the oracle here).  Every call runs on a
NaN-poisoned h and y with sentinel bands."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import Guarded, assert_within, bf16_bits_to_f64, dev, say

pytestmark = pytest.mark.gpu


class Layer:
    """Device grids of one MoE shape."""

    def __init__(self, shape: synth.MoEShape, cfg: int, layer: int = 0):
        self.shape = shape
        self.gu = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_GATE_UP, shape.E, 2 * shape.I, shape.hidden)
        self.dn = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_DOWN, shape.E, shape.hidden, shape.I)
        self.dgu = [dev(self.gu.codes), dev(self.gu.scales), dev(self.gu.biases)]
        self.ddn = [dev(self.dn.codes), dev(self.dn.scales), dev(self.dn.biases)]

    def run(self, x, ids, p, f32=False, h=None, y=None):
        """One layer call into Guarded h (bf16) and y, poisoned first; returns (h bits, y)."""
        sh = self.shape
        h = h or Guarded((sh.topk, sh.I), False)
        y = y or Guarded((sh.hidden,), f32)
        h.poison()
        y.poison()
        qmm.qmm_moe_layer(dev(x), *self.dgu, *self.ddn, dev(np.asarray(ids, np.int32)),
                          dev(np.asarray(p, np.float32)), h.t, y.t)
        torch.cuda.synchronize()
        return h.values(), y.values()

    def two_calls(self, x, ids, p, f32=False):
        """The same token through the two qmm_moe_gather calls (stage 2 on stage 1's h)."""
        sh = self.shape
        h = Guarded((sh.topk, sh.I), False)
        y = Guarded((sh.hidden,), f32)
        idd = dev(np.asarray(ids, np.int32))
        qmm.qmm_moe_gather(qmm.QMM_MOE_GATE_UP_SWIGLU, dev(x), *self.dgu, idd, h.t)
        qmm.qmm_moe_gather(qmm.QMM_MOE_DOWN_COMBINE, h.t, *self.ddn, idd, y.t,
                           expert_w=dev(np.asarray(p, np.float32)))
        torch.cuda.synchronize()
        return h.values(), y.values()


def check_call(L: Layer, x, ids, p, f32=False, oracle=True):
    hg, yg = L.run(x, ids, p, f32)
    h2, y2 = L.two_calls(x, ids, p, f32)
    assert np.array_equal(hg, h2), "h differs from the two-call path"
    assert np.array_equal(yg, y2) if f32 else np.array_equal(yg.view(np.uint16), y2.view(np.uint16)), \
        "y differs from the two-call path"
    if oracle:
        h, th = orc.moe_gate_up(x, L.gu.codes, L.gu.scales, L.gu.biases, ids, 2 * L.shape.I)
        # the GPU's bf16 h against the oracle: the stated bound, plus the rounding of a value
        # within it to bf16 (at most 2^-8 of its magnitude)
        assert_within(bf16_bits_to_f64(hg), h, th + (np.abs(h) + th) * 2.0 ** -8, "layer h")


def test_35B_layer_over_consecutive_calls():
    """Six tokens in a row, fresh x and routing each."""
    sh = synth.MOE_35B
    say(f"[moe layer] {sh.name}, 6 calls")
    L = Layer(sh, synth.CFG_MOE)
    for s in range(6):
        x = synth.gen_x(synth.CFG_MOE, 0, s, 1, sh.hidden)[0]
        ids, p = synth.gen_routing(synth.CFG_MOE, 0, s, sh.E, sh.topk)
        check_call(L, x, ids, p, oracle=(s == 0))


SHAPES = [
    synth.MoEShape("hidden 512, 12 experts, I 128, top-4", 512, 12, 128, 4),      # stage 1 and 2 on 16 lanes/row
    synth.MoEShape("hidden 1024, 16 experts, I 1024, top-3", 1024, 16, 1024, 3),  # 3 waves per block
    synth.MoEShape("hidden 5120, 16 experts, I 2048, top-10", 5120, 16, 2048, 10),  # 5 chunks, 2 slots per wave
    synth.MoEShape("hidden 2560, 6 experts, I 768, top-1", 2560, 6, 768, 1),
]


@pytest.mark.parametrize("shape", SHAPES, ids=["h512-I128-top4", "h1024-I1024-top3", "h5120-I2048-top10",
                                               "h2560-I768-top1"])
def test_layer_shapes(shape):
    say(f"[moe layer] {shape.name}")
    L = Layer(shape, synth.CFG_TEST, 3)
    for s in range(2):
        x = synth.gen_x(synth.CFG_TEST, 3, s, 1, shape.hidden)[0]
        ids, p = synth.gen_routing(synth.CFG_TEST, 3, s, shape.E, shape.topk)
        check_call(L, x, ids, p, f32=(s == 1))


def test_layer_no_expert_ids_and_repeats():
    shape = SHAPES[0]
    L = Layer(shape, synth.CFG_TEST, 4)
    x = synth.gen_x(synth.CFG_TEST, 4, 0, 1, shape.hidden)[0]
    for ids in ([3, -1, shape.E, 3], [-1, -1, -1, -1], [5, 5, 5, 5]):
        say(f"[moe layer] ids {ids}")
        p = np.array([0.4, 0.3, 0.2, 0.1], np.float32)
        hg, _ = L.run(x, ids, p)
        for k, e in enumerate(ids):
            if not 0 <= e < shape.E:
                assert np.all(hg[k] == 0)
        check_call(L, x, ids, p)


def test_layer_graph_replays_with_eager_calls_between():
    """Four tokens captured in one graph (each its own h and y), replayed three times with an
    eager call between replays; every replay equals the eager result."""
    sh = synth.MOE_35B
    say("[moe layer] graph replays")
    L = Layer(sh, synth.CFG_MOE, 1)
    n = 4
    xs = [dev(synth.gen_x(synth.CFG_MOE, 1, s, 1, sh.hidden)[0]) for s in range(n)]
    rt = [synth.gen_routing(synth.CFG_MOE, 1, s, sh.E, sh.topk) for s in range(n)]
    ids = [dev(np.asarray(r[0], np.int32)) for r in rt]
    ps = [dev(np.asarray(r[1], np.float32)) for r in rt]
    hs = [Guarded((sh.topk, sh.I), False) for _ in range(n)]
    ys = [Guarded((sh.hidden,), False) for _ in range(n)]
    want = [L.two_calls(synth.gen_x(synth.CFG_MOE, 1, s, 1, sh.hidden)[0], rt[s][0], rt[s][1]) for s in range(n)]
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        for s in range(n):  # once eagerly outside the capture
            qmm.qmm_moe_layer(xs[s], *L.dgu, *L.ddn, ids[s], ps[s], hs[s].t, ys[s].t, stream=st)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for s in range(n):
                qmm.qmm_moe_layer(xs[s], *L.dgu, *L.ddn, ids[s], ps[s], hs[s].t, ys[s].t, stream=st)
    torch.cuda.synchronize()
    x_other = synth.gen_x(synth.CFG_MOE, 1, 99, 1, sh.hidden)[0]
    r_other = synth.gen_routing(synth.CFG_MOE, 1, 99, sh.E, sh.topk)
    for rep in range(3):
        for s in range(n):
            hs[s].poison()
            ys[s].poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(n):
            assert np.array_equal(hs[s].values(), want[s][0]), (rep, s)
            assert np.array_equal(ys[s].values(), want[s][1]), (rep, s)
        check_call(L, x_other, r_other[0], r_other[1], oracle=False)  # eager, between replays
