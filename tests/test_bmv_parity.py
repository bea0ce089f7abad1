"""GPU parity of the small-batch path (u4 group 64, K a multiple of 512 up to 8192:
activations on the matrix cores, the weights streamed once per 16 or 32 rows; taken for
2 <= M <= 32 and above where the prefill GEMM would be slower) against the fp64 oracle.

Acceptance as for the decode GEMV (the oracle's `tolerance`, propagated for SwiGLU): the
path rounds no weight, so the bound without the bf16-weight term applies.  Also: a row's
result does not depend on the other rows of the batch (bit for bit), fused outputs equal
the unfused projection on the same row slice, y(2x) = 2 y(x) exactly, all-zero codes and
biases or an all-zero input give exact zeros, and no write lands outside an output."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import Guarded, assert_within, dev, dev_weight, rne_bits_of, say

pytestmark = pytest.mark.gpu


def run_linear(x, w, f32=True, lin_bias=None):
    y = Guarded((x.shape[0], w.rows), f32)
    c, s, b = dev_weight(w)
    qmm.qmm_linear(dev(x), c, s, b, y.t, lin_bias=None if lin_bias is None else dev(lin_bias))
    torch.cuda.synchronize()
    return y.values()


def run_qkv(x, w, q_out, kv_out, f32=True, lin_bias=None):
    M = x.shape[0]
    outs = [Guarded((M, n), f32) for n in (q_out, kv_out, kv_out)]
    c, s, b = dev_weight(w)
    qmm.qmm_fused_qkv(dev(x), c, s, b, outs[0].t, outs[1].t, outs[2].t,
                      lin_bias=None if lin_bias is None else dev(lin_bias))
    torch.cuda.synchronize()
    return [o.values() for o in outs]


def run_gate_up(x, w, I, f32=True):
    h = Guarded((x.shape[0], I), f32)
    c, s, b = dev_weight(w)
    qmm.qmm_fused_gate_up_swiglu(dev(x), c, s, b, h.t)
    torch.cuda.synchronize()
    return h.values()


# every K the path is built for, ragged row counts (units of 16 rows), M across one and
# two 16-row passes
@pytest.mark.parametrize("M,K,N", [(2, 1024, 16), (3, 2048, 70), (5, 3072, 33), (8, 4096, 48), (16, 5120, 200),
                                   (17, 6144, 21), (31, 7168, 40), (32, 8192, 64), (4, 5120, 1)])
def test_linear(M, K, N):
    say(f"[bmv] linear M={M} K={K} N={N}")
    w = synth.gen_weight(synth.CFG_TEST, 400 + M, synth.PROJ_LINEAR, N, K, bias="uniform")
    x = synth.gen_x(synth.CFG_TEST, 400 + M, 0, M, K, magnitude="varied")
    lb = synth.gen_lin_bias(synth.CFG_TEST, 400 + M, N)
    y, t = orc.linear(x, w.codes, w.scales, w.biases, lb)
    got = run_linear(x, w, lin_bias=lb)
    assert_within(got, y, t, f"linear M={M} K={K} N={N}")
    # bf16 output = RNE of the fp32 output
    assert np.array_equal(run_linear(x, w, f32=False, lin_bias=lb), rne_bits_of(got))


@pytest.mark.parametrize("M,K,q_out,kv_out", [(2, 5120, 5120, 1024), (7, 2048, 40, 8), (24, 1024, 17, 3)])
def test_fused_qkv(M, K, q_out, kv_out):
    say(f"[bmv] qkv M={M} K={K} q={q_out} kv={kv_out}")
    rows = q_out + 2 * kv_out
    w = synth.gen_weight(synth.CFG_TEST, 410 + M, synth.PROJ_QKV, rows, K)
    x = synth.gen_x(synth.CFG_TEST, 410 + M, 0, M, K)
    lb = synth.gen_lin_bias(synth.CFG_TEST, 410 + M, rows)
    (q, k, v), (tq, tk, tv) = orc.fused_qkv(x, w.codes, w.scales, w.biases, q_out, kv_out, lb)
    g = run_qkv(x, w, q_out, kv_out, lin_bias=lb)
    for got, ref, tol, nm in zip(g, (q, k, v), (tq, tk, tv), "QKV"):
        assert_within(got, ref, tol, f"qkv M={M} {nm}")
    # fused = unfused on the same row slices
    full = run_linear(x, w, lin_bias=lb)
    assert np.array_equal(g[0], full[:, :q_out])
    assert np.array_equal(g[1], full[:, q_out:q_out + kv_out])
    assert np.array_equal(g[2], full[:, q_out + kv_out:])


@pytest.mark.parametrize("M,K,I", [(2, 5120, 13824), (6, 1024, 1), (13, 2048, 71), (32, 4096, 40)])
def test_gate_up_swiglu(M, K, I):
    say(f"[bmv] gate+up M={M} K={K} I={I}")
    w = synth.gen_weight(synth.CFG_TEST, 420 + M, synth.PROJ_GATE_UP, 2 * I, K)
    x = synth.gen_x(synth.CFG_TEST, 420 + M, 0, M, K, magnitude="varied")
    h, th = orc.gate_up_swiglu(x, w.codes, w.scales, w.biases, I)
    got = run_gate_up(x, w, I)
    assert_within(got, h, th, f"gate+up M={M} K={K} I={I}")
    # silu(gate) * up of the unfused rows
    lin = run_linear(x, w)
    g, u = lin[:, :I], lin[:, I:]
    ref = (g / (1.0 + np.exp(-g))) * u
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_rows_do_not_depend_on_the_batch():
    """Within the small-batch regime (3 <= M <= 32 here) a row's result is the same bits
    whatever the other rows are."""
    K, N = 5120, 96
    say("[bmv] batch invariance")
    w = synth.gen_weight(synth.CFG_TEST, 430, synth.PROJ_LINEAR, N, K)
    x = synth.gen_x(synth.CFG_TEST, 430, 0, 20, K)
    full = run_linear(x, w)                      # two passes of 16 rows
    assert np.array_equal(run_linear(x[3:6], w), full[3:6])
    assert np.array_equal(run_linear(x[16:20], w), full[16:20])
    assert np.array_equal(run_linear(x[[7, 2, 19]], w), full[[7, 2, 19]])


def test_exact_cases():
    K, N, M = 2048, 48, 5
    say("[bmv] exact zeros and linearity")
    w = synth.gen_weight(synth.CFG_TEST, 431, synth.PROJ_LINEAR, N, K)
    x = synth.gen_x(synth.CFG_TEST, 431, 0, M, K)
    zero = synth.U4Weight(np.zeros_like(w.codes), w.scales, np.zeros_like(w.biases))
    assert np.all(run_linear(x, zero) == 0.0)
    assert np.all(run_linear(np.zeros_like(x), w) == 0.0)
    x2 = orc.f32_to_bf16_bits(2.0 * orc.bf16_to_f64(x))
    assert np.array_equal(run_linear(x2, w), 2.0 * run_linear(x, w))


def test_14B_shapes_against_sampled_rows():
    """The 14B layer's fused gate+up at M = 16: sampled output columns against the oracle
    computed on those weight rows only."""
    M, K, I = 16, 5120, 13824
    say(f"[bmv] 14B gate+up M={M}")
    w = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_GATE_UP, 2 * I, K)
    x = synth.gen_x(synth.CFG_14B, 0, 0, M, K)
    got = run_gate_up(x, w, I)
    cols = np.random.default_rng(5).choice(I, 48, replace=False)
    rows = np.concatenate([cols, I + cols])
    sub = synth.U4Weight(w.codes[rows], w.scales[rows], w.biases[rows])
    h, th = orc.gate_up_swiglu(x, sub.codes, sub.scales, sub.biases, len(cols))
    assert_within(got[:, cols], h, th, "14B gate+up sampled")


def test_many_passes_14B_qkv():
    """M = 96 on the 14B fused QKV (7168 rows): six 16-row passes, which the dispatch
    prefers to the 28-tile prefill GEMM.  Sampled columns against the oracle on those
    rows; the rows of the last pass equal the same rows of a one-pass call bit for bit."""
    M, sh = 96, synth.DENSE_14B
    say(f"[bmv] 14B qkv M={M}")
    w = synth.gen_weight(synth.CFG_14B, 1, synth.PROJ_QKV, sh.qkv_rows, sh.K)
    x = synth.gen_x(synth.CFG_14B, 1, 0, M, sh.K)
    q, k, v = run_qkv(x, w, sh.q_out, sh.kv_out)
    full = np.concatenate([q, k, v], axis=1)
    cols = np.sort(np.random.default_rng(6).choice(sh.qkv_rows, 64, replace=False))
    sub = synth.U4Weight(w.codes[cols], w.scales[cols], w.biases[cols])
    y, t = orc.linear(x, sub.codes, sub.scales, sub.biases)
    assert_within(full[:, cols], y, t, "14B qkv M=96 sampled")
    q2, k2, v2 = run_qkv(x[80:96], w, sh.q_out, sh.kv_out)
    assert np.array_equal(np.concatenate([q2, k2, v2], axis=1), full[80:96])


def test_ragged_last_pass():
    """M = 37 (passes of 16, 16 and 5 rows) on a 24B-shaped gate+up slice."""
    M, K, I = 37, 5120, 300
    say(f"[bmv] gate+up M={M} K={K} I={I}")
    w = synth.gen_weight(synth.CFG_TEST, 440, synth.PROJ_GATE_UP, 2 * I, K)
    x = synth.gen_x(synth.CFG_TEST, 440, 0, M, K)
    h, th = orc.gate_up_swiglu(x, w.codes, w.scales, w.biases, I)
    assert_within(run_gate_up(x, w, I), h, th, f"gate+up M={M}")


@pytest.mark.parametrize("M", [2, 16, 33])
@pytest.mark.parametrize("sh", [synth.ROPE_14B, synth.ROPE_GATED], ids=["14B", "gated"])
def test_fused_qkv_rope(sh, M):
    """Fused QKV + split + rotary embedding through the small-batch kernel (units of 8
    rotating pairs): against the oracle, and bf16 = RNE(fp32)."""
    say(f"[bmv] qkv+rope {sh.name} M={M}")
    max_pos = 4096
    w = synth.gen_weight(synth.CFG_TEST, 450 + M, synth.PROJ_QKV, sh.rows, sh.K)
    lb = synth.gen_lin_bias(synth.CFG_TEST, 450 + M, sh.rows)
    x = synth.gen_x(synth.CFG_TEST, 450 + M, 0, M, sh.K)
    pos = synth.gen_positions(synth.CFG_TEST, 450 + M, M, max_pos, contiguous=False)
    tab = synth.gen_rope_table(max_pos, sh.rot, sh.base)

    def run(f32):
        outs = [Guarded((M, sh.n_q, sh.head_dim), f32), Guarded((M, sh.n_kv, sh.head_dim), f32),
                Guarded((M, sh.n_kv, sh.head_dim), f32)]
        g = Guarded((M, sh.n_q, sh.head_dim), f32) if sh.q_gate else None
        qmm.qmm_fused_qkv_rope(dev(x), dev(w.codes), dev(w.scales), dev(w.biases), outs[0].t, outs[1].t, outs[2].t,
                               dev(np.asarray(pos, np.int32)), dev(tab), sh.rot, gate=g.t if g else None,
                               lin_bias=dev(lb))
        torch.cuda.synchronize()
        return outs[0].values(), (g.values() if g else None), outs[1].values(), outs[2].values()

    got = run(True)
    ref, tol = orc.qkv_rope(x, w.codes, w.scales, w.biases, sh.n_q, sh.n_kv, sh.head_dim, sh.q_gate, sh.rot,
                            pos, tab, lb)
    for name, g, r, t in zip(("q", "gate", "k", "v"), got, ref, tol):
        if r is None:
            assert g is None
            continue
        assert_within(g, r, t, f"{sh.name} M={M} {name}")
    for g32, g16 in zip(got, run(False)):
        if g32 is not None:
            assert np.array_equal(g16, rne_bits_of(g32))
