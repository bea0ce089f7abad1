"""A decode step in few launches (qmm_step_plan / qmm_step_run) against the per-call entry
points and the fp64 oracle.

The step kernel computes every projection with the per-call decode arithmetic for its K
(the same lanes, chunks, operation order and K-slice order), so each output must equal
the per-call result bit for bit; outputs that do not depend on another GPU result are
also checked against the oracle at the stated rule.  A projection that reads another
one's output (the down projection reading its layer's h) runs in a later launch of the same
run; the chained results are compared with the per-call chain, and a down projection fed the
oracle's own rounded h is checked against the oracle.  Graph replays of a step are
compared with its eager run, with NaN poisoning of every output between replays."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import Guarded, assert_within, dev, dev_weight, say

pytestmark = pytest.mark.gpu


class Plan:
    """A planned step: the projections (host) and the plan (device)."""

    def __init__(self, projs):
        self.projs = projs
        n = qmm.qmm_step_plan_bytes(projs)
        assert n > 0
        self.mem = torch.empty(n, dtype=torch.uint8, device="cuda")
        qmm.qmm_step_plan(projs, self.mem)

    def run(self, stream=None):
        qmm.qmm_step_run(self.projs, self.mem, stream=stream)


def plan_of(projs):
    return Plan(projs)


def bits_equal(a, b, what):
    """Bit patterns equal: fp32 values (held as float64) or bf16 bit patterns (uint16)."""
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float64:
        av, bv = a.astype(np.float32).view(np.uint32), b.astype(np.float32).view(np.uint32)
    else:
        av, bv = a, b
    bad = np.flatnonzero(av.ravel() != bv.ravel())
    assert bad.size == 0, f"{what}: {bad.size} elements differ from the per-call result, first {bad[:5].tolist()}"


class Layer:
    """One dense layer's weights on the device (fused QKV, fused gate+up, down)."""

    def __init__(self, sh, cfg, L):
        self.qkv = synth.gen_weight(cfg, L, synth.PROJ_QKV, sh.qkv_rows, sh.K)
        self.gu = synth.gen_weight(cfg, L, synth.PROJ_GATE_UP, 2 * sh.I, sh.K)
        self.dn = synth.gen_weight(cfg, L, synth.PROJ_DOWN, sh.K, sh.I)
        self.dqkv, self.dgu, self.ddn = dev_weight(self.qkv), dev_weight(self.gu), dev_weight(self.dn)


def test_14B_step_one_launch_equals_per_call_and_oracle():
    """The 14B-shaped decode step (fused QKV + fused gate+up+SwiGLU, K = 5120) in one launch."""
    sh = synth.DENSE_14B
    say("[step] 14B: fused QKV + gate+up in one launch")
    qkv = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_QKV, sh.qkv_rows, sh.K)
    gu = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_GATE_UP, 2 * sh.I, sh.K)
    x1 = synth.gen_x(synth.CFG_14B, 0, 0, 1, sh.K)
    x2 = synth.gen_x(synth.CFG_14B, 0, 1, 1, sh.K)
    dq, dg = dev_weight(qkv), dev_weight(gu)
    xd1, xd2 = dev(x1), dev(x2)
    for f32 in (True, False):
        q, k, v = (Guarded((1, n), f32) for n in (sh.q_out, sh.kv_out, sh.kv_out))
        h = Guarded((1, sh.I), f32)
        plan = plan_of([qmm.step_fused_qkv(xd1, *dq, q.t, k.t, v.t), qmm.step_gate_up_swiglu(xd2, *dg, h.t)])
        plan.run()
        torch.cuda.synchronize()
        got = [o.values() for o in (q, k, v, h)]
        # per-call
        rq, rk, rv = (Guarded((1, n), f32) for n in (sh.q_out, sh.kv_out, sh.kv_out))
        rh = Guarded((1, sh.I), f32)
        qmm.qmm_fused_qkv(xd1, *dq, rq.t, rk.t, rv.t)
        qmm.qmm_fused_gate_up_swiglu(xd2, *dg, rh.t)
        torch.cuda.synchronize()
        for a, b, nm in zip(got, (rq.values(), rk.values(), rv.values(), rh.values()), ("Q", "K", "V", "h")):
            bits_equal(a, b, f"14B step {nm} ({'f32' if f32 else 'bf16'})")
        if f32:
            (oq, ok, ov), (tq, tk, tv) = orc.fused_qkv(x1, qkv.codes, qkv.scales, qkv.biases, sh.q_out, sh.kv_out)
            oh, th = orc.gate_up_swiglu(x2, gu.codes, gu.scales, gu.biases, sh.I)
            for g_, r_, t_, nm in zip(got, (oq, ok, ov, oh), (tq, tk, tv, th), ("Q", "K", "V", "h")):
                assert_within(g_, r_, t_, f"14B step {nm}")


def dense_step_projs(layers, sh, xd, outs):
    """The projections of a dense step in list order: QKV and gate+up of layer l + 1 before
    the down projection of layer l (which waits for its layer's gate+up)."""
    projs, gu_index = [], {}
    L = len(layers)
    order = []
    for l in range(L):
        order += [("qkv", l), ("gu", l)]
        if l >= 1:
            order.append(("dn", l - 1))
    order.append(("dn", L - 1))
    for kind, l in order:
        lay, (q, k, v, h, y) = layers[l], outs[l]
        if kind == "qkv":
            projs.append(qmm.step_fused_qkv(xd, *lay.dqkv, q.t, k.t, v.t))
        elif kind == "gu":
            gu_index[l] = len(projs)
            projs.append(qmm.step_gate_up_swiglu(xd, *lay.dgu, h.t))
        else:
            projs.append(qmm.step_linear(h.t, *lay.ddn, y.t, wait_for=gu_index[l]))
    return projs


def test_24B_step_with_down_waiting_for_h():
    """Three 24B-dense-shaped layers in one run (two launches): each layer's down projection
    (K = 32768, split over 8 waves) reads the h its layer's gate+up wrote in the same run.
    The first launch (QKV and gate+up of three layers, 107520 positions, 620 MB) is a long
    launch, which the planner runs at two blocks per CU on a 256-CU GPU."""
    sh = synth.DENSE_24B
    L = 3
    layers = [Layer(sh, synth.CFG_24B, l) for l in range(L)]
    x = synth.gen_x(synth.CFG_24B, 0, 0, 1, sh.K)
    xd = dev(x)
    outs = [(Guarded((1, sh.q_out), True), Guarded((1, sh.kv_out), True), Guarded((1, sh.kv_out), True),
             Guarded((1, sh.I), False), Guarded((1, sh.K), True)) for _ in range(L)]
    plan = plan_of(dense_step_projs(layers, sh, xd, outs))
    for rep in range(3):
        say(f"[step] 24B x {L} layers, run {rep}")
        for o in outs:
            for g in o:
                g.poison()
        plan.run()
        torch.cuda.synchronize()
        for l, lay in enumerate(layers):
            q, k, v, h, y = (g.values() for g in outs[l])
            rq, rk, rv = (Guarded((1, n), True) for n in (sh.q_out, sh.kv_out, sh.kv_out))
            rh, ry = Guarded((1, sh.I), False), Guarded((1, sh.K), True)
            qmm.qmm_fused_qkv(xd, *lay.dqkv, rq.t, rk.t, rv.t)
            qmm.qmm_fused_gate_up_swiglu(xd, *lay.dgu, rh.t)
            qmm.qmm_linear(rh.t, *lay.ddn, ry.t)
            torch.cuda.synchronize()
            for a, b, nm in zip((q, k, v, h, y), (rq.values(), rk.values(), rv.values(), rh.values(), ry.values()),
                                "QKVhy"):
                bits_equal(a, b, f"24B layer {l} {nm} (run {rep})")
    # layer 0 against the oracle (the down on the GPU's h is covered by the per-call chain)
    (oq, ok, ov), (tq, tk, tv) = orc.fused_qkv(x, layers[0].qkv.codes, layers[0].qkv.scales, layers[0].qkv.biases,
                                              sh.q_out, sh.kv_out)
    q, k, v = (g.values() for g in outs[0][:3])
    for g_, r_, t_, nm in zip((q, k, v), (oq, ok, ov), (tq, tk, tv), "QKV"):
        assert_within(g_, r_, t_, f"24B step layer 0 {nm}")


def test_step_down_projection_on_the_oracles_h():
    """The K-split launch of the step (24B down, K = 32768 over 8 waves) on an h that the
    oracle made: checked against the oracle at the stated rule."""
    sh = synth.DENSE_24B
    dn = synth.gen_weight(synth.CFG_24B, 5, synth.PROJ_DOWN, sh.K, sh.I)
    gu = synth.gen_weight(synth.CFG_24B, 5, synth.PROJ_GATE_UP, 2 * sh.I, sh.K)
    x = synth.gen_x(synth.CFG_24B, 5, 0, 1, sh.K)
    rh, _ = orc.gate_up_swiglu(x, gu.codes, gu.scales, gu.biases, sh.I)
    hb = orc.f32_to_bf16_bits(rh)
    y = Guarded((1, sh.K), True)
    hd, dw = dev(hb), dev_weight(dn)        # the plan keeps pointers: keep the tensors alive
    plan = plan_of([qmm.step_linear(hd, *dw, y.t)])
    plan.run()
    torch.cuda.synchronize()
    ry, ty = orc.linear(hb, dn.codes, dn.scales, dn.biases)
    assert_within(y.values(), ry, ty, "step down on the oracle's h")


# the K of each link of a chain of plain projections: link i reads link i - 1's bf16 output
# (so its row count is the next K); single-slice and K-split shapes, a ragged last row count
CHAIN_K = [576, 1088, 5184, 8192, 2048, 45056]
CHAIN_LAST_N = 777


def test_dependency_chain_of_projections():
    """Six projections, each waiting for the one before it (x = its bf16 output), with
    K-split and single-slice shapes mixed and additive biases: one run (six launches)
    equals the per-call chain bit for bit."""
    Ns = CHAIN_K[1:] + [CHAIN_LAST_N]
    ws, bs, outs = [], [], []
    xin = dev(synth.gen_x(synth.CFG_TEST, 60, 0, 1, CHAIN_K[0]))
    for i, (K, N) in enumerate(zip(CHAIN_K, Ns)):
        w = synth.gen_weight(synth.CFG_TEST, 60 + i, synth.PROJ_LINEAR, N, K, scale_lo=0.0005, scale_hi=0.002,
                             bias="uniform")
        ws.append(dev_weight(w))
        bs.append(dev(synth.gen_lin_bias(synth.CFG_TEST, 60 + i, N)))
        outs.append(torch.full((N,), 0x7FC0, dtype=torch.int16, device="cuda"))
    projs = [qmm.step_linear(xin if i == 0 else outs[i - 1], *ws[i], outs[i], lin_bias=bs[i], wait_for=i - 1)
             for i in range(len(CHAIN_K))]
    plan = plan_of(projs)
    plan.run()
    torch.cuda.synchronize()
    ref_in = xin
    for i in range(len(CHAIN_K)):
        r = torch.empty_like(outs[i])
        qmm.qmm_linear(ref_in.view(1, -1), *ws[i], r.view(1, -1), lin_bias=bs[i])
        torch.cuda.synchronize()
        bits_equal(outs[i].cpu().numpy().view(np.uint16), r.cpu().numpy().view(np.uint16), f"chain link {i}")
        ref_in = r
    say(f"[step] chain of {len(CHAIN_K)} projections equal to the per-call chain")


MIXED = [
    # (kind, K, rows / (q_out, kv_out), bias, f32): every epilogue at single-slice and K-split K
    ("qkv", 576, (33, 7), True, True),
    ("lin", 36864, 130, True, True),      # 8 waves, 5 chunks per lane
    ("qkv", 8192, (64, 32), True, False),
    ("qkv", 45056, (12, 2), False, True),
    ("gu", 1088, 17, False, True),
    ("gu", 8192, 48, False, False),
    ("gu", 65536, 33, False, True),
    ("lin", 2048, 301, True, True),
    ("lin", 13824, 5120, False, True),
]


def test_mixed_epilogues_in_one_launch():
    """Fused QKV, gate+up and plain projections at single-slice and K-split K (8 waves at 4 and
    5 chunks per lane, 16 waves), bf16 and fp32 outputs, with and without additive bias, all
    independent, in one run (one launch per kind): each equals its per-call result bit for
    bit and the oracle at the stated rule."""
    projs, checks, keep = [], [], []       # keep: device inputs the plan points to
    for i, (kind, K, r, bias, f32) in enumerate(MIXED):
        x = synth.gen_x(synth.CFG_TEST, 70 + i, 0, 1, K)
        xd = dev(x)
        if kind == "qkv":
            q_out, kv_out = r
            rows = q_out + 2 * kv_out
            w = synth.gen_weight(synth.CFG_TEST, 70 + i, synth.PROJ_QKV, rows, K)
            lb = synth.gen_lin_bias(synth.CFG_TEST, 70 + i, rows) if bias else None
            o = [Guarded((1, n), f32) for n in (q_out, kv_out, kv_out)]
            dw, dlb = dev_weight(w), None if lb is None else dev(lb)
            keep += [dw, dlb]
            projs.append(qmm.step_fused_qkv(xd, *dw, *(g.t for g in o), lin_bias=dlb))
            checks.append((kind, x, xd, w, lb, o, (q_out, kv_out), f32))
        elif kind == "gu":
            I = r
            w = synth.gen_weight(synth.CFG_TEST, 70 + i, synth.PROJ_GATE_UP, 2 * I, K)
            o = [Guarded((1, I), f32)]
            dw = dev_weight(w)
            keep.append(dw)
            projs.append(qmm.step_gate_up_swiglu(xd, *dw, o[0].t))
            checks.append((kind, x, xd, w, None, o, I, f32))
        else:
            N = r
            w = synth.gen_weight(synth.CFG_TEST, 70 + i, synth.PROJ_LINEAR, N, K)
            lb = synth.gen_lin_bias(synth.CFG_TEST, 70 + i, N) if bias else None
            o = [Guarded((1, N), f32)]
            dw, dlb = dev_weight(w), None if lb is None else dev(lb)
            keep += [dw, dlb]
            projs.append(qmm.step_linear(xd, *dw, o[0].t, lin_bias=dlb))
            checks.append((kind, x, xd, w, lb, o, N, f32))
    plan = plan_of(projs)
    plan.run()
    torch.cuda.synchronize()
    for kind, x, xd, w, lb, o, r, f32 in checks:
        got = [g.values() for g in o]
        ref = [Guarded(g.t.shape, f32) for g in o]
        dw = dev_weight(w)
        if kind == "qkv":
            qmm.qmm_fused_qkv(xd.view(1, -1), *dw, *(g.t for g in ref), lin_bias=None if lb is None else dev(lb))
        elif kind == "gu":
            qmm.qmm_fused_gate_up_swiglu(xd.view(1, -1), *dw, ref[0].t)
        else:
            qmm.qmm_linear(xd.view(1, -1), *dw, ref[0].t, lin_bias=None if lb is None else dev(lb))
        torch.cuda.synchronize()
        for a, g in zip(got, ref):
            bits_equal(a, g.values(), f"{kind} K={x.shape[1]}")
        if f32:
            if kind == "qkv":
                rr, tt = orc.fused_qkv(x, w.codes, w.scales, w.biases, r[0], r[1], lb)
            elif kind == "gu":
                rr, tt = orc.gate_up_swiglu(x, w.codes, w.scales, w.biases, r)
                rr, tt = (rr,), (tt,)
            else:
                rr, tt = orc.linear(x, w.codes, w.scales, w.biases, lb)
                rr, tt = (rr,), (tt,)
            for a, b, t in zip(got, rr, tt):
                assert_within(a, b, t, f"step {kind} K={x.shape[1]}")


def test_graph_replays_of_a_step_equal_its_eager_run():
    """A 24B-shaped two-layer step (two launches) captured in a HIP graph and replayed five
    times, with every output NaN-poisoned and unrelated eager work between the replays: each
    replay equals the eager run bit for bit."""
    sh = synth.DENSE_24B
    L = 2
    layers = [Layer(sh, synth.CFG_24B, 10 + l) for l in range(L)]
    xd = dev(synth.gen_x(synth.CFG_24B, 10, 0, 1, sh.K))
    outs = [(Guarded((1, sh.q_out), True), Guarded((1, sh.kv_out), True), Guarded((1, sh.kv_out), True),
             Guarded((1, sh.I), False), Guarded((1, sh.K), True)) for _ in range(L)]
    plan = plan_of(dense_step_projs(layers, sh, xd, outs))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        plan.run(stream=s)
    torch.cuda.synchronize()
    eager = [[g.values() for g in o] for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run(stream=s)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(5):
        for o in outs:
            for b in o:
                b.poison()
        junk.mul_(1.0001)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            for a, b, nm in zip((b_.values() for b_ in outs[l]), eager[l], "QKVhy"):
                bits_equal(a, b, f"replay {rep} layer {l} {nm}")
    say("[step] five graph replays equal the eager run")
