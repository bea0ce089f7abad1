"""GPU parity of the prefill path (M > 8: LDS dequant + MFMA GEMM) against the fp64 oracle.

Same acceptance rule as the decode path: the stated 1e-3 * sum|x w| (propagated for
SwiGLU), on the fp32 output before bf16 rounding.  The prefill design rounds each
dequantized weight to bf16 before the MFMA (tiles dequantized to bf16 in LDS); at short
K (< 512) the check adds that rounding's exact bound, sum |x| |w - bf16(w)|
(`bf16_term`), and from K = 512 up, the 14B shapes included, it uses the stated rule
alone.  The GEMM is therefore not bit-equal to the decode GEMV; both are checked against
the oracle, a GEMM row is also compared with the GEMV on that row, and the fused
gate+up GEMM equals SwiGLU of the two unfused GEMM projections."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import bf16_term, Guarded, assert_within, dev, dev_weight, rne_bits_of, say

pytestmark = pytest.mark.gpu


def run_qkv(x, w, q_out, kv_out, f32=True, lin_bias=None):
    M = x.shape[0]
    outs = [Guarded((M, n), f32) for n in (q_out, kv_out, kv_out)]
    c, s, b = dev_weight(w)
    qmm.qmm_fused_qkv(dev(x), c, s, b, outs[0].t, outs[1].t, outs[2].t,
                      lin_bias=None if lin_bias is None else dev(lin_bias))
    torch.cuda.synchronize()
    return [o.values() for o in outs]


def run_linear(x, w, f32=True):
    y = Guarded((x.shape[0], w.rows), f32)
    c, s, b = dev_weight(w)
    qmm.qmm_linear(dev(x), c, s, b, y.t)
    torch.cuda.synchronize()
    return y.values()


def run_gate_up(x, w, I, f32=True):
    h = Guarded((x.shape[0], I), f32)
    c, s, b = dev_weight(w)
    qmm.qmm_fused_gate_up_swiglu(dev(x), c, s, b, h.t)
    torch.cuda.synchronize()
    return h.values()


def test_prefill_fused_qkv_14B_shape():
    sh = synth.DENSE_14B
    M = synth.PREFILL_M
    say(f"[gemm] fused QKV prefill M={M} K={sh.K} rows={sh.qkv_rows}")
    w = synth.gen_weight(synth.CFG_PREFILL, 0, synth.PROJ_QKV, sh.qkv_rows, sh.K)
    x = synth.gen_x(synth.CFG_PREFILL, 0, 0, M, sh.K)
    (q, k, v), (tq, tk, tv) = orc.fused_qkv(x, w.codes, w.scales, w.biases, sh.q_out, sh.kv_out)
    g = run_qkv(x, w, sh.q_out, sh.kv_out)
    for got, ref, tol, nm in zip(g, (q, k, v), (tq, tk, tv), "QKV"):
        assert_within(got, ref, tol, f"prefill {nm}")
    gb = run_qkv(x, w, sh.q_out, sh.kv_out, f32=False)
    for got32, got16, nm in zip(g, gb, "QKV"):
        assert np.array_equal(got16, rne_bits_of(got32)), f"{nm}: bf16 output != RNE(fp32 output)"
    # a GEMM row against the decode GEMV on that row (both within the oracle's bound)
    for m in (0, 1000, M - 1):
        gv = run_qkv(x[m:m + 1], w, sh.q_out, sh.kv_out)
        for part, got, ref, tol in zip(gv, g, (q, k, v), (tq, tk, tv)):
            assert np.all(np.abs(part[0] - got[m]) <= 2 * tol[m])


def test_prefill_gate_up_14B_shape():
    sh = synth.DENSE_14B
    M = synth.PREFILL_M
    say(f"[gemm] fused gate+up prefill M={M} K={sh.K} I={sh.I}")
    w = synth.gen_weight(synth.CFG_PREFILL, 0, synth.PROJ_GATE_UP, 2 * sh.I, sh.K)
    x = synth.gen_x(synth.CFG_PREFILL, 0, 0, M, sh.K)
    h, th = orc.gate_up_swiglu(x, w.codes, w.scales, w.biases, sh.I)
    g = run_gate_up(x, w, sh.I)
    assert_within(g, h, th, "prefill h")
    gb = run_gate_up(x, w, sh.I, f32=False)
    assert np.array_equal(gb, rne_bits_of(g)), "bf16 output != RNE(fp32 output)"
    # the fused gate+up GEMM against SwiGLU of the two unfused GEMM projections ("The
    # Cathedral Doubled Itself", the two fusions: one matmul over [gate; up] then
    # SiLU * multiply): the gate and up accumulators are the unfused values bit for bit,
    # so only the fp32 evaluation of silu(g) * u separates them
    gl = run_linear(x, w.slice_rows(0, sh.I))
    ul = run_linear(x, w.slice_rows(sh.I, 2 * sh.I))
    ref = orc.swiglu(gl, ul)
    rel = np.abs(g - ref) / np.maximum(np.abs(ref), 1e-30)
    say(f"  fused vs swiglu(unfused): max rel {rel.max():.3g}")
    assert np.all(np.abs(g - ref) <= 2.0 ** -20 * np.abs(ref) + 1e-30)


RAGGED = [
    # (name, M, K, q_out, kv_out)
    ("M=9 K=512", 9, 512, 64, 32),
    ("M=100 K=576 rows 111", 100, 576, 47, 32),
    ("M=300 K=64 rows 300", 300, 64, 100, 100),
    ("M=257 K=1088 rows 520", 257, 1088, 256, 132),
    ("doubled-Q M=40", 40, synth.DOUBLED_Q.K, synth.DOUBLED_Q.q_out, synth.DOUBLED_Q.kv_out),
]


@pytest.mark.parametrize("name,M,K,q_out,kv_out", RAGGED, ids=[r[0] for r in RAGGED])
def test_prefill_ragged_qkv(name, M, K, q_out, kv_out):
    say(f"[gemm] {name}")
    w = synth.gen_weight(synth.CFG_TEST, 100 + M, synth.PROJ_QKV, q_out + 2 * kv_out, K, bias="uniform")
    x = synth.gen_x(synth.CFG_TEST, 100 + M, 0, M, K)
    lb = synth.gen_lin_bias(synth.CFG_TEST, 100 + M, q_out + 2 * kv_out)
    (q, k, v), (tq, tk, tv) = orc.fused_qkv(x, w.codes, w.scales, w.biases, q_out, kv_out, lb,
                                            bf16_weights=bf16_term(M, K))
    g = run_qkv(x, w, q_out, kv_out, lin_bias=lb)
    for got, ref, tol, nm in zip(g, (q, k, v), (tq, tk, tv), "QKV"):
        assert_within(got, ref, tol, f"{name} {nm}")


@pytest.mark.parametrize("M,K,I", [(9, 512, 1), (33, 2048, 129), (300, 640, 200), (520, 5120, 300)])
def test_prefill_ragged_gate_up(M, K, I):
    say(f"[gemm] gate+up M={M} K={K} I={I}")
    w = synth.gen_weight(synth.CFG_TEST, 200 + M, synth.PROJ_GATE_UP, 2 * I, K)
    x = synth.gen_x(synth.CFG_TEST, 200 + M, 0, M, K, magnitude="varied")
    h, th = orc.gate_up_swiglu(x, w.codes, w.scales, w.biases, I, bf16_weights=bf16_term(M, K, heavy_tailed=True))
    assert_within(run_gate_up(x, w, I), h, th, f"gate+up M={M} K={K} I={I}")


def test_prefill_linear_down_shape_and_determinism():
    """A 24B-dense down projection shape (K = 32768) at M = 64, run twice."""
    M, K, N = 64, 32768, 512
    say(f"[gemm] linear M={M} K={K} N={N}")
    w = synth.gen_weight(synth.CFG_TEST, 300, synth.PROJ_DOWN, N, K)
    x = synth.gen_x(synth.CFG_TEST, 300, 0, M, K)
    y, t = orc.linear(x, w.codes, w.scales, w.biases)
    a = run_linear(x, w)
    assert_within(a, y, t, "down M=64")
    assert np.array_equal(a, run_linear(x, w))


def test_prefill_exact_cases():
    """Weights exactly representable in bf16 (codes 0 or 8 +- powers of two with bias
    -8*scale): the GEMM's bf16 rounding of w is exact, and zero input gives zero."""
    M, K, N = 64, 1024, 96
    w = synth.gen_weight(synth.CFG_TEST, 301, synth.PROJ_LINEAR, N, K)
    rng = np.random.default_rng(7)
    allowed = np.array([0, 4, 6, 7, 8, 9, 10, 12], np.uint64)
    q = allowed[rng.integers(0, len(allowed), size=(N, K))]
    words = np.zeros((N, K // 8), np.uint64)
    for j in range(8):
        words |= q[:, j::8] << np.uint64(4 * j)
    w = synth.U4Weight(words.astype(np.uint32), w.scales, w.biases)
    x = synth.gen_x(synth.CFG_TEST, 301, 0, M, K)
    y, t = orc.linear(x, w.codes, w.scales, w.biases)
    assert_within(run_linear(x, w), y, t, "exactly representable weights")
    assert np.all(run_linear(np.zeros_like(x), w) == 0.0)
