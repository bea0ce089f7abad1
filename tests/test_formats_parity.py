"""GPU parity of the other formats of the affine family (code width, group size) against
the fp64 oracle: projections, fused QKV, fused gate+up and the routed-expert gather, in
decode (GEMV) and prefill (GEMM), through the *_fmt calls of the C ABI."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import bf16_term, Guarded, assert_within, dev, rne_bits_of, say

pytestmark = pytest.mark.gpu

FP8 = qmm.QMM_FP8_E4M3
FORMATS = [(4, 32), (4, 128), (8, 64), (8, 32), (6, 64), (6, 128), (3, 64), (3, 32), (2, 64), (2, 128),
           (FP8, 64), (FP8, 128)]


def ob(bits):
    """The oracle's and the generator's name of an ABI format code."""
    return orc.E4M3 if bits == FP8 else bits


def W(bits, G, rows, K, layer, index=0):
    return synth.gen_weight(synth.CFG_TEST, layer, synth.PROJ_LINEAR, rows, K, index=index, bits=ob(bits), group=G)


def lin(bits, G, x, w, N, f32=True, lb=None):
    M = x.shape[0]
    y = Guarded((M, N), f32)
    qmm.qmm_linear_fmt(bits, G, dev(x), dev(w.codes), dev(w.scales), dev(w.biases), y.t,
                       lin_bias=None if lb is None else dev(lb))
    torch.cuda.synchronize()
    return y.values()


@pytest.mark.parametrize("bits,G", FORMATS)
@pytest.mark.parametrize("M,K,N", [(1, 512, 300), (3, 5120, 200), (1, 8192, 130), (2, 64 * 45, 77),
                                   (40, 1024, 260), (300, 640, 129)])
def test_linear_formats(bits, G, M, K, N):
    if K % G:
        pytest.skip("K is not a whole number of groups")
    say(f"[fmt] linear u{bits} g{G} M={M} K={K} N={N}")
    w = W(bits, G, N, K, 1)
    lb = synth.gen_lin_bias(synth.CFG_TEST, 1, N)
    x = synth.gen_x(synth.CFG_TEST, 1, M, M, K)
    y, t = orc.linear(x, w.codes, w.scales, w.biases, lb, bf16_weights=bf16_term(M, K, bits == FP8), bits=ob(bits))
    g = lin(bits, G, x, w, N, lb=lb)
    assert_within(g, y, t, f"u{bits} g{G} linear M={M} K={K}")
    assert np.array_equal(lin(bits, G, x, w, N, f32=False, lb=lb), rne_bits_of(g))
    if M == 2:
        # both rows in one launch of the GEMV, each equal to its own M = 1 call
        for m in range(2):
            assert np.array_equal(lin(bits, G, x[m:m + 1], w, N, lb=lb)[0], g[m]), f"row {m}"


@pytest.mark.parametrize("bits,G", FORMATS)
@pytest.mark.parametrize("M", [1, 64])
def test_fused_qkv_and_gate_up_formats(bits, G, M):
    K, q_out, kv_out, I = 1024, 256, 64, 192
    say(f"[fmt] fused u{bits} g{G} M={M}")
    x = synth.gen_x(synth.CFG_TEST, 2, M, M, K)
    wq = W(bits, G, q_out + 2 * kv_out, K, 2)
    (q, k, v), (tq, tk, tv) = orc.fused_qkv(x, wq.codes, wq.scales, wq.biases, q_out, kv_out,
                                            bf16_weights=bf16_term(M, K, bits == FP8), bits=ob(bits))
    gq, gk, gv = Guarded((M, q_out), True), Guarded((M, kv_out), True), Guarded((M, kv_out), True)
    qmm.qmm_fused_qkv_fmt(bits, G, dev(x), dev(wq.codes), dev(wq.scales), dev(wq.biases), gq.t, gk.t, gv.t)
    wg = W(bits, G, 2 * I, K, 3)
    h, th = orc.gate_up_swiglu(x, wg.codes, wg.scales, wg.biases, I, bf16_weights=bf16_term(M, K, bits == FP8), bits=ob(bits))
    gh = Guarded((M, I), True)
    qmm.qmm_fused_gate_up_swiglu_fmt(bits, G, dev(x), dev(wg.codes), dev(wg.scales), dev(wg.biases), gh.t)
    torch.cuda.synchronize()
    for got, ref, tol, name in ((gq, q, tq, "q"), (gk, k, tk, "k"), (gv, v, tv, "v"), (gh, h, th, "h")):
        assert_within(got.values(), ref, tol, f"u{bits} g{G} {name} M={M}")


@pytest.mark.parametrize("bits,G", FORMATS)
def test_moe_gather_formats(bits, G):
    E, hidden, I, topk = 6, 512, 128, 3
    say(f"[fmt] moe u{bits} g{G}")
    gu = synth.gen_expert_grid(synth.CFG_TEST, 4, synth.PROJ_MOE_GATE_UP, E, 2 * I, hidden, bits=ob(bits), group=G)
    dn = synth.gen_expert_grid(synth.CFG_TEST, 4, synth.PROJ_MOE_DOWN, E, hidden, I, bits=ob(bits), group=G)
    x = synth.gen_x(synth.CFG_TEST, 4, 0, 1, hidden)[0]
    ids = np.array([4, -1, 1], np.int32)
    p = np.array([0.5, 0.2, 0.3], np.float32)
    h, th = orc.moe_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * I, bits=ob(bits))
    g1 = Guarded((topk, I), True)
    qmm.qmm_moe_gather_fmt(bits, G, qmm.QMM_MOE_GATE_UP_SWIGLU, dev(x), dev(gu.codes), dev(gu.scales),
                           dev(gu.biases), dev(ids), g1.t)
    hb = orc.f32_to_bf16_bits(h)
    y, ty = orc.moe_down_combine(hb, dn.codes, dn.scales, dn.biases, ids, p, bits=ob(bits))
    g2 = Guarded((hidden,), True)
    qmm.qmm_moe_gather_fmt(bits, G, qmm.QMM_MOE_DOWN_COMBINE, dev(hb), dev(dn.codes), dev(dn.scales),
                           dev(dn.biases), dev(ids), g2.t, expert_w=dev(p))
    torch.cuda.synchronize()
    assert_within(g1.values(), h, th, f"u{bits} g{G} moe stage 1")
    assert_within(g2.values(), y, ty, f"u{bits} g{G} moe stage 2")


@pytest.mark.parametrize("M", [1, 40])
def test_fmt_at_u4_g64_is_the_plain_call_bit_for_bit(M):
    K, N = 1024, 300
    w = W(4, 64, N, K, 5)
    x = synth.gen_x(synth.CFG_TEST, 5, 0, M, K)
    a = lin(4, 64, x, w, N)
    b = Guarded((M, N), True)
    qmm.qmm_linear(dev(x), dev(w.codes), dev(w.scales), dev(w.biases), b.t)
    torch.cuda.synchronize()
    assert np.array_equal(a, b.values())


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8, FP8])
def test_largest_K_per_width(bits):
    """The deepest K split of the decode kernel at each width's largest K, and the GEMM."""
    K = 65536 if bits in (2, 4) else 49152
    N = 48
    w = W(bits, 64, N, K, 6)
    for M in (1, 16):
        say(f"[fmt] u{bits} K={K} M={M}")
        x = synth.gen_x(synth.CFG_TEST, 6, M, M, K)
        y, t = orc.linear(x, w.codes, w.scales, w.biases, bf16_weights=bf16_term(M, K, bits == FP8), bits=ob(bits))
        assert_within(lin(bits, 64, x, w, N), y, t, f"u{bits} K={K} M={M}")


def test_wide_codes_past_their_largest_K_are_rejected():
    x = torch.zeros((1, 49216), dtype=torch.int16, device="cuda")
    for bits in (3, 6, 8, FP8):
        w = W(bits, 64, 1, 49216, 7)
        y = torch.zeros((1, 1), dtype=torch.float32, device="cuda")
        with pytest.raises(qmm.QmmError) as e:
            qmm.qmm_linear_fmt(bits, 64, x, dev(w.codes), dev(w.scales), dev(w.biases), y)
        assert e.value.status == qmm.STATUS["QMM_ERR_SHAPE"]


@pytest.mark.parametrize("M", [1, 16])
def test_every_fp8_code_decodes_to_its_e4m3_value(M):
    """Row r holds the 254 finite e4m3 patterns at inputs 0..253 (scale 1, bias 0); x is
    one-hot at input k, so y[r] is exactly the value of code k: the GPU's conversion is the
    format's definition (decode and prefill, where the value is also a bf16 operand)."""
    K, G = 256, 64
    codes8 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F] + [0, 0], np.uint8)
    words = np.tile(codes8.view("<u4").astype(np.uint32), (4, 1))
    one = orc.f32_to_bf16_bits(np.ones(1))[0]
    s_ = np.full((4, K // G), one, np.uint16)
    b_ = np.zeros((4, K // G), np.uint16)
    ks = np.arange(M) * 15 % 254
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = one
    w = synth.U4Weight(words, s_, b_, 8)
    y = lin(FP8, G, x, w, 4)
    expect = orc.e4m3_to_f64(codes8[ks])
    say(f"[fmt] every fp8 code, M={M}")
    assert np.array_equal(y, np.repeat(expect[:, None], 4, axis=1))
