"""A 20-step decode loop over 24B-dense-shaped layers (fused QKV, fused gate+up+SwiGLU,
down projection), with a fresh x every step and the same output buffers reused.

Every step of every layer is compared with the oracle at the stated rule; odd steps
first poison the outputs with NaN so a stale value cannot pass, and sentinel bands
catch writes outside the buffers.  The down projection is checked on its own input:
each step uploads the oracle's h rounded to bf16 and runs the down projection on it
(M = 1, K = 32768, N = 5120), so no GPU value ever becomes an oracle input.  The down
projection chained on the GPU's own h runs too, as in a real step; it is checked only
for finite values and intact sentinel bands (its input is the GPU's, not the oracle's)."""
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
    h = Guarded((1, sh.I), False)                # bf16 h, read by the chained down projection
    hf = Guarded((1, sh.I), True)                # fp32 h of the same call, for the SwiGLU check
    y = Guarded((1, sh.K), True)                 # chained down (GPU h): NaN and sentinel guard only
    yi = Guarded((1, sh.K), True)                # down on the oracle's rounded h: value check
    hin = torch.empty((1, sh.I), dtype=torch.int16, device="cuda")

    for L, (qkv, gu, dn, dqkv, dgu, ddn) in enumerate(layers):
        say(f"[loop] layer {L}: oracle")
        (rq, rk, rv), (tq, tk, tv) = orc.fused_qkv(X, qkv.codes, qkv.scales, qkv.biases, sh.q_out, sh.kv_out)
        rh, th = orc.gate_up_swiglu(X, gu.codes, gu.scales, gu.biases, sh.I)
        hb = orc.f32_to_bf16_bits(rh)            # [20, I]: the down projection's input per step
        ry, ty = orc.linear(hb, dn.codes, dn.scales, dn.biases)
        for step in range(STEPS):
            if step % 2:
                for o in (q, k, v, h, hf, y, yi):
                    o.poison()
            xd = dev(xs[step])
            hin.copy_(dev(hb[step:step + 1]))
            qmm.qmm_fused_qkv(xd, *dqkv, q.t, k.t, v.t)
            qmm.qmm_fused_gate_up_swiglu(xd, *dgu, h.t)
            qmm.qmm_fused_gate_up_swiglu(xd, *dgu, hf.t)
            qmm.qmm_linear(h.t, *ddn, y.t)
            qmm.qmm_linear(hin, *ddn, yi.t)
            torch.cuda.synchronize()
            say(f"[loop] layer {L} step {step}")
            assert_within(q.values()[0], rq[step], tq[step], "Q")
            assert_within(k.values()[0], rk[step], tk[step], "K")
            assert_within(v.values()[0], rv[step], tv[step], "V")
            assert_within(hf.values()[0], rh[step], th[step], "h")
            assert_within(yi.values()[0], ry[step], ty[step], "down")
            assert np.all(np.isfinite(y.values())), "chained down: non-finite output"
