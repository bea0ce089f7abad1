"""A 20-step decode loop over 24B-dense-shaped layers (fused QKV, fused gate+up+SwiGLU,
down projection), with a fresh x every step and the same output buffers reused.

Every step of every layer is compared with the oracle; odd steps first poison the
outputs with NaN so a stale value cannot pass, and sentinel bands catch writes
outside the buffers.  The down projection reads the GPU's own bf16 h, so its bound
adds |W_down| times the largest difference a bf16 rounding of an h inside its own
tolerance can make (computed from the oracle's h alone)."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import Guarded, assert_within, dev, dev_weight, say

pytestmark = pytest.mark.gpu

STEPS = 20
LAYERS = 2   # of the shape's 40; every layer has the full 24B-dense shapes


def test_twenty_step_decode_loop():
    sh = synth.DENSE_24B
    cfg = synth.CFG_24B
    layers = []
    for L in range(LAYERS):
        qkv = synth.gen_weight(cfg, L, synth.PROJ_QKV, sh.qkv_rows, sh.K)
        gu = synth.gen_weight(cfg, L, synth.PROJ_GATE_UP, 2 * sh.I, sh.K)
        dn = synth.gen_weight(cfg, L, synth.PROJ_DOWN, sh.K, sh.I)
        layers.append((qkv, gu, dn, dev_weight(qkv), dev_weight(gu), dev_weight(dn)))
    xs = [synth.gen_x(cfg, 0, step, 1, sh.K) for step in range(STEPS)]
    X = np.concatenate(xs)                       # [20, K]: the oracle runs all steps at once

    q = Guarded((1, sh.q_out), True)
    k = Guarded((1, sh.kv_out), True)
    v = Guarded((1, sh.kv_out), True)
    h = Guarded((1, sh.I), False)                # bf16 h, read by the down projection
    hf = Guarded((1, sh.I), True)                # fp32 h of the same call, for the SwiGLU check
    y = Guarded((1, sh.K), True)

    for L, (qkv, gu, dn, dqkv, dgu, ddn) in enumerate(layers):
        say(f"[loop] layer {L}: oracle")
        (rq, rk, rv), (tq, tk, tv) = orc.fused_qkv(X, qkv.codes, qkv.scales, qkv.biases, sh.q_out, sh.kv_out)
        rh, th = orc.gate_up_swiglu(X, gu.codes, gu.scales, gu.biases, sh.I)
        # down reads bf16(h_gpu); the oracle feeds RNE(h_oracle) and widens the bound
        herr = orc.bf16_input_error(rh, th)
        ry, ty = orc.linear_with_input_error(orc.f32_to_bf16_bits(rh), dn.codes, dn.scales, dn.biases, herr)
        for step in range(STEPS):
            if step % 2:
                for o in (q, k, v, h, hf, y):
                    o.poison()
            xd = dev(xs[step])
            qmm.qmm_fused_qkv(xd, *dqkv, q.t, k.t, v.t)
            qmm.qmm_fused_gate_up_swiglu(xd, *dgu, h.t)
            qmm.qmm_fused_gate_up_swiglu(xd, *dgu, hf.t)
            qmm.qmm_linear(h.t, *ddn, y.t)
            torch.cuda.synchronize()
            say(f"[loop] layer {L} step {step}")
            assert_within(q.values()[0], rq[step], tq[step], "Q")
            assert_within(k.values()[0], rk[step], tk[step], "K")
            assert_within(v.values()[0], rv[step], tv[step], "V")
            assert_within(hf.values()[0], rh[step], th[step], "h")
            assert_within(y.values()[0], ry[step], ty[step], "down")
