"""GPU parity of the routed-expert gather (decode) against the fp64 oracle.

Stage 1 (gathered gate+up+SwiGLU) and stage 2 (gathered down + weighted combine)
are each checked on the same inputs as the oracle: stage 2 reads an h made by the
oracle and rounded to bf16, never the GPU's stage-1 output."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import Guarded, assert_within, dev, rne_bits_of, say

pytestmark = pytest.mark.gpu


def make_grids(shape: synth.MoEShape, layer: int, cfg: int):
    gu = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_GATE_UP, shape.E, 2 * shape.I, shape.hidden)
    dn = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_DOWN, shape.E, shape.hidden, shape.I)
    return gu, dn


def run_stage1(x, grid, ids, I, f32=True):
    out = Guarded((len(ids), I), f32)
    qmm.qmm_moe_gather(qmm.QMM_MOE_GATE_UP_SWIGLU, dev(x), dev(grid.codes), dev(grid.scales), dev(grid.biases),
                       dev(np.asarray(ids, np.int32)), out.t)
    torch.cuda.synchronize()
    return out.values()


def run_stage2(h_bits, grid, ids, p, rows, f32=True):
    out = Guarded((rows,), f32)
    qmm.qmm_moe_gather(qmm.QMM_MOE_DOWN_COMBINE, dev(h_bits), dev(grid.codes), dev(grid.scales), dev(grid.biases),
                       dev(np.asarray(ids, np.int32)), out.t, expert_w=dev(np.asarray(p, np.float32)))
    torch.cuda.synchronize()
    return out.values()


SMALL = synth.MoEShape("small MoE (hidden 512, 12 experts, I 128, top-4)", 512, 12, 128, 4)


@pytest.mark.parametrize("shape", [SMALL, synth.MOE_35B], ids=["small", "35B-A3B-shaped"])
def test_moe_two_stages_match_oracle(shape):
    say(f"[moe] {shape.name}")
    cfg = synth.CFG_MOE if shape is synth.MOE_35B else synth.CFG_TEST
    gu, dn = make_grids(shape, 0, cfg)
    x = synth.gen_x(cfg, 0, 0, 1, shape.hidden)[0]
    ids, p = synth.gen_routing(cfg, 0, 0, shape.E, shape.topk)
    h, th = orc.moe_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * shape.I)
    g1 = run_stage1(x, gu, ids, shape.I)
    assert_within(g1, h, th, "stage 1 h")
    g1b = run_stage1(x, gu, ids, shape.I, f32=False)
    assert np.array_equal(g1b, rne_bits_of(g1))
    h_bits = orc.f32_to_bf16_bits(h)   # the oracle's own h, rounded, feeds both sides
    y, ty = orc.moe_down_combine(h_bits, dn.codes, dn.scales, dn.biases, ids, p)
    g2 = run_stage2(h_bits, dn, ids, p, shape.hidden)
    assert_within(g2, y, ty, "stage 2 y")


def test_moe_no_expert_ids_and_repeats():
    shape = SMALL
    gu, dn = make_grids(shape, 1, synth.CFG_TEST)
    x = synth.gen_x(synth.CFG_TEST, 1, 0, 1, shape.hidden)[0]
    ids = np.array([3, -1, shape.E, 3, 11], np.int32)     # out-of-range ids and a repeat
    p = np.array([0.3, 0.2, 0.1, 0.25, 0.15], np.float32)
    say("[moe] ids with no expert and repeats")
    h, th = orc.moe_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * shape.I)
    g1 = run_stage1(x, gu, ids, shape.I)
    assert np.all(g1[1] == 0) and np.all(g1[2] == 0)
    assert_within(g1, h, th, "stage 1 with gaps")
    assert np.array_equal(g1[0], g1[3])
    h_bits = orc.f32_to_bf16_bits(h)
    y, ty = orc.moe_down_combine(h_bits, dn.codes, dn.scales, dn.biases, ids, p)
    assert_within(run_stage2(h_bits, dn, ids, p, shape.hidden), y, ty, "stage 2 with gaps")


def test_moe_single_expert_equals_dense_calls():
    """topk = 1, p = 1: stage 1 equals qmm_fused_gate_up_swiglu and stage 2 equals
    qmm_linear on that expert's slice of the grid, bit for bit."""
    shape = SMALL
    gu, dn = make_grids(shape, 2, synth.CFG_TEST)
    x = synth.gen_x(synth.CFG_TEST, 2, 0, 1, shape.hidden)
    for e in (0, 7, shape.E - 1):
        g1 = run_stage1(x[0], gu, [e], shape.I)
        h = Guarded((1, shape.I), True)
        ew = gu.codes[e], gu.scales[e], gu.biases[e]
        qmm.qmm_fused_gate_up_swiglu(dev(x), dev(ew[0]), dev(ew[1]), dev(ew[2]), h.t)
        torch.cuda.synchronize()
        assert np.array_equal(g1, h.values()), e
        hb = rne_bits_of(g1)
        g2 = run_stage2(hb, dn, [e], [1.0], shape.hidden)
        y = Guarded((1, shape.hidden), True)
        qmm.qmm_linear(dev(hb), dev(dn.codes[e]), dev(dn.scales[e]), dev(dn.biases[e]), y.t)
        torch.cuda.synchronize()
        assert np.array_equal(g2, y.values()[0]), e


def test_moe_combine_order_invariance():
    shape = SMALL
    gu, dn = make_grids(shape, 3, synth.CFG_TEST)
    rng = np.random.default_rng(3)
    h_bits = synth.to_bf16_bits(rng.standard_normal((shape.topk, shape.I)).astype(np.float32))
    ids, p = synth.gen_routing(synth.CFG_TEST, 3, 0, shape.E, shape.topk)
    a = run_stage2(h_bits, dn, ids, p, shape.hidden)
    perm = [2, 0, 3, 1]
    b = run_stage2(h_bits[perm], dn, ids[perm], p[perm], shape.hidden)
    y, ty = orc.moe_down_combine(h_bits, dn.codes, dn.scales, dn.biases, ids, p)
    assert_within(a, y, ty, "order a")
    assert_within(b, y, ty, "order b")
