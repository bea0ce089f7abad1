"""qmm_moe_prefill_noalloc (the routed-experts prefill for callers that cannot allocate:
its routing and stage-2 products live in the library's own device scratch array) against
the existing entry point with a caller workspace, qmm_moe_prefill after qmm_moe_route, on
the same inputs: the same kernels, so the outputs must agree bit for bit.  Two calls in a
row per path, the second on a smaller batch, so stale scratch contents from the first
call cannot pass; the no-allocation path's outputs are NaN-poisoned before each call."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import Guarded, assert_within, dev, say

pytestmark = pytest.mark.gpu

SMALL = synth.MoEShape("small MoE prefill (hidden 320, 8 experts, I 192, top-2)", 320, 8, 192, 2)


def both_stages(shape, cfg, layer, M, skew):
    gu = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_GATE_UP, shape.E, 2 * shape.I, shape.hidden)
    dn = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_DOWN, shape.E, shape.hidden, shape.I)
    ids, p = synth.gen_prefill_routing(cfg, layer, M, shape.E, shape.topk, skew=skew)
    x = synth.gen_x(cfg, layer, 0, M, shape.hidden)
    h_in = synth.gen_x(cfg, layer, 1, M * shape.topk, shape.I).reshape(M, shape.topk, shape.I)
    return gu, dn, ids, p, x, h_in


def run_pair(gu, dn, ids, p, x, h_in, shape):
    """Stage 1 and stage 2 through both entry points; returns ((h_ws, y_ws), (h_na, y_na))."""
    M, topk = ids.shape
    did, dp = dev(np.ascontiguousarray(ids, np.int32)), dev(np.asarray(p, np.float32))
    dx, dh = dev(x), dev(h_in)
    g1 = [dev(a) for a in (gu.codes, gu.scales, gu.biases)]
    g2 = [dev(a) for a in (dn.codes, dn.scales, dn.biases)]
    # existing entry point: caller workspace, routed first
    ws = torch.empty(qmm.qmm_moe_prefill_workspace_bytes(M, topk, shape.E, shape.hidden), dtype=torch.uint8,
                     device="cuda")
    h_ws = Guarded((M, topk, shape.I), True)
    y_ws = Guarded((M, shape.hidden), True)
    qmm.qmm_moe_route(did, shape.E, ws)
    qmm.qmm_moe_prefill(qmm.QMM_MOE_GATE_UP_SWIGLU, dx, *g1, did, ws, h_ws.t)
    qmm.qmm_moe_prefill(qmm.QMM_MOE_DOWN_COMBINE, dh, *g2, did, ws, y_ws.t, expert_w=dp)
    # the no-allocation entry point
    h_na = Guarded((M, topk, shape.I), True)
    y_na = Guarded((M, shape.hidden), True)
    h_na.poison()
    y_na.poison()
    qmm.qmm_moe_prefill_noalloc(qmm.QMM_MOE_GATE_UP_SWIGLU, dx, *g1, did, h_na.t)
    qmm.qmm_moe_prefill_noalloc(qmm.QMM_MOE_DOWN_COMBINE, dh, *g2, did, y_na.t, expert_w=dp)
    torch.cuda.synchronize()
    return (h_ws.values(), y_ws.values()), (h_na.values(), y_na.values())


CASES = [
    # (name, shape, cfg, layer, M first, M second, skew): the routed path (many pairs and
    # few pairs per expert) and the pair-by-pair path, each twice with a smaller batch
    ("several routing tiles per expert", SMALL, synth.CFG_TEST, 40, 2000, 700, 1.0),
    ("35B-A3B shape, few pairs per expert", synth.MOE_35B, synth.CFG_MOE, 0, 256, 96, 0.5),
    ("35B-A3B shape, pair by pair", synth.MOE_35B, synth.CFG_MOE, 1, 32, 9, 0.5),
]


@pytest.mark.parametrize("name,shape,cfg,layer,m1,m2,skew", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_entry_point(name, shape, cfg, layer, m1, m2, skew):
    for M in (m1, m2):
        say(f"[noalloc] {name}: M={M} ({M * shape.topk} pairs)")
        gu, dn, ids, p, x, h_in = both_stages(shape, cfg, layer, M, skew)
        (h_ws, y_ws), (h_na, y_na) = run_pair(gu, dn, ids, p, x, h_in, shape)
        assert np.array_equal(h_na.view(np.uint32), h_ws.view(np.uint32)), "stage 1 differs"
        assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), "stage 2 differs"


def test_noalloc_against_the_oracle():
    shape = SMALL
    M = 300
    gu, dn, ids, p, x, h_in = both_stages(shape, synth.CFG_TEST, 41, M, 1.0)
    _, (h_na, y_na) = run_pair(gu, dn, ids, p, x, h_in, shape)
    h, th = orc.moe_prefill_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * shape.I, bf16_weights=True)
    assert_within(h_na, h, th, "noalloc stage 1")
    y, ty = orc.moe_prefill_down_combine(h_in, dn.codes, dn.scales, dn.biases, ids, p, bf16_weights=True)
    assert_within(y_na, y, ty, "noalloc stage 2")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    shape = synth.MOE_35B
    M = 2048                       # stage 2: 16384 pairs x 2048 rows of fp32 products > 64 MiB
    assert qmm.qmm_moe_prefill_workspace_bytes(M, shape.topk, shape.E, shape.hidden) > qmm.QMM_NOALLOC_SCRATCH_BYTES
    h = torch.zeros((M, shape.topk, shape.I), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((shape.E, shape.hidden, shape.I // 8), dtype=torch.int32, device="cuda")
    sb = torch.zeros((shape.E, shape.hidden, shape.I // 64), dtype=torch.int16, device="cuda")
    ids = torch.zeros((M, shape.topk), dtype=torch.int32, device="cuda")
    w = torch.zeros((M, shape.topk), dtype=torch.float32, device="cuda")
    y = torch.zeros((M, shape.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(qmm.QmmError, match="QMM_ERR_SHAPE"):
        qmm.qmm_moe_prefill_noalloc(qmm.QMM_MOE_DOWN_COMBINE, h, codes, sb, sb, ids, y, expert_w=w)
