"""GPU parity of the fused QKV + split + rotary embedding (qmm_fused_qkv_rope) against the
fp64 oracle, in every regime (the GEMV at M = 1 and, where the small-batch kernel does
not apply, up to M = 8; the small-batch kernel; the prefill GEMM), full and partial
rotary, with and without the per-head output gate; plus two exact identities: at angle
zero the outputs are the plain fused QKV outputs bit for bit, and bf16 output =
RNE(fp32 output)."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import bf16_term, Guarded, assert_within, dev, rne_bits_of, say

pytestmark = pytest.mark.gpu

SMALL = synth.RopeShape("small QKV + RoPE (hidden 1024, 6 q / 2 kv heads x 128, full rotary)",
                        1024, 6, 2, 128, False, 128, 1.0e4)
SMALL_GATED = synth.RopeShape("small gated QKV + RoPE (hidden 512, 3 q heads x 256 with gate, 1 kv head, "
                              "rotary 64)", 512, 3, 1, 256, True, 64, 1.0e7)
MAX_POS = 4096


def weights(sh, cfg, layer):
    w = synth.gen_weight(cfg, layer, synth.PROJ_QKV, sh.rows, sh.K)
    lb = synth.gen_lin_bias(cfg, layer, sh.rows)
    return w, lb


class Outs:
    def __init__(self, sh, M, f32):
        self.q = Guarded((M, sh.n_q, sh.head_dim), f32)
        self.k = Guarded((M, sh.n_kv, sh.head_dim), f32)
        self.v = Guarded((M, sh.n_kv, sh.head_dim), f32)
        self.g = Guarded((M, sh.n_q, sh.head_dim), f32) if sh.q_gate else None

    def values(self):
        return (self.q.values(), self.g.values() if self.g else None, self.k.values(), self.v.values())


def run(sh, x, w, lb, pos, tab, f32=True):
    M = x.shape[0]
    o = Outs(sh, M, f32)
    qmm.qmm_fused_qkv_rope(dev(x), dev(w.codes), dev(w.scales), dev(w.biases), o.q.t, o.k.t, o.v.t,
                           dev(np.asarray(pos, np.int32)), dev(tab), sh.rot, gate=o.g.t if o.g else None,
                           lin_bias=None if lb is None else dev(lb))
    torch.cuda.synchronize()
    return o.values()


def check(sh, cfg, layer, M, contiguous=True, sample=None, with_bias=True):
    w, lb = weights(sh, cfg, layer)
    lb = lb if with_bias else None
    x = synth.gen_x(cfg, layer, 0, M, sh.K)
    pos = synth.gen_positions(cfg, layer, M, MAX_POS, contiguous)
    tab = synth.gen_rope_table(MAX_POS, sh.rot, sh.base)
    got = run(sh, x, w, lb, pos, tab)
    rows = np.arange(M) if sample is None else sample
    ref, tol = orc.qkv_rope(x[rows], w.codes, w.scales, w.biases, sh.n_q, sh.n_kv, sh.head_dim, sh.q_gate,
                            sh.rot, pos[rows], tab, lb, bf16_weights=bf16_term(M, sh.K))
    for name, g, r, t in zip(("q", "gate", "k", "v"), got, ref, tol):
        if r is None:
            assert g is None
            continue
        assert_within(g[rows], r, t, f"{sh.name} M={M} {name}")
    bf = run(sh, x, w, lb, pos, tab, f32=False)
    for g32, g16 in zip(got, bf):
        if g32 is not None:
            assert np.array_equal(g16, rne_bits_of(g32))


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("sh", [SMALL, SMALL_GATED], ids=["full", "gated"])
def test_rope_decode_matches_oracle(sh, M):
    say(f"[rope] decode {sh.name} M={M}")
    check(sh, synth.CFG_TEST, 1, M, contiguous=False)


@pytest.mark.parametrize("M", [9, 300])
@pytest.mark.parametrize("sh", [SMALL, SMALL_GATED], ids=["full", "gated"])
def test_rope_prefill_matches_oracle(sh, M):
    say(f"[rope] prefill {sh.name} M={M}")
    check(sh, synth.CFG_TEST, 2, M)


def test_rope_without_bias_and_partial_rotary_decode():
    sh = synth.RopeShape("QKV + RoPE without bias, rotary 32 of 64", 512, 4, 2, 64, False, 32, 1.0e4)
    say(f"[rope] {sh.name}")
    check(sh, synth.CFG_TEST, 3, 2, with_bias=False)
    check(sh, synth.CFG_TEST, 3, 40, with_bias=False)


@pytest.mark.parametrize("M", [1, 64])
def test_rope_at_angle_zero_equals_fused_qkv_bit_for_bit(M):
    """cos = 1, sin = 0 at every position: q/k/v are the fused QKV outputs, split into heads."""
    sh = SMALL
    w, lb = weights(sh, synth.CFG_TEST, 4)
    x = synth.gen_x(synth.CFG_TEST, 4, 0, M, sh.K)
    tab = np.concatenate([np.ones((8, sh.rot // 2)), np.zeros((8, sh.rot // 2))], axis=1).astype(np.float32)
    pos = np.arange(M, dtype=np.int32) % 8
    q, _, k, v = run(sh, x, w, lb, pos, tab)
    qo, ko = sh.n_q * sh.head_dim, sh.n_kv * sh.head_dim
    fq, fk, fv = Guarded((M, qo), True), Guarded((M, ko), True), Guarded((M, ko), True)
    qmm.qmm_fused_qkv(dev(x), dev(w.codes), dev(w.scales), dev(w.biases), fq.t, fk.t, fv.t, lin_bias=dev(lb))
    torch.cuda.synchronize()
    say(f"[rope] angle zero == fused QKV, M={M}")
    assert np.array_equal(q.reshape(M, -1), fq.values())
    assert np.array_equal(k.reshape(M, -1), fk.values())
    assert np.array_equal(v.reshape(M, -1), fv.values())


def test_rope_positions_outside_the_table_are_clamped():
    sh = SMALL
    w, lb = weights(sh, synth.CFG_TEST, 5)
    x = synth.gen_x(synth.CFG_TEST, 5, 0, 4, sh.K)
    tab = synth.gen_rope_table(64, sh.rot, sh.base)
    pos = np.array([-5, 63, 64, 100000], np.int32)
    got = run(sh, x, w, lb, pos, tab)
    ref, tol = orc.qkv_rope(x, w.codes, w.scales, w.biases, sh.n_q, sh.n_kv, sh.head_dim, False, sh.rot,
                            np.clip(pos, 0, 63), tab, lb)
    say("[rope] clamped positions")
    for g, r, t in zip(got, ref, tol):
        if r is not None:
            assert_within(g, r, t, "clamped positions")


@pytest.mark.parametrize("sh", [synth.ROPE_14B, synth.ROPE_GATED], ids=["14B", "gated"])
def test_rope_full_size_decode_and_sampled_prefill(sh):
    """The workload shapes: decode M=1, and prefill at 2048 tokens checked on sampled tokens."""
    say(f"[rope] {sh.name}: decode")
    check(sh, synth.CFG_14B, 0, 1)
    say(f"[rope] {sh.name}: prefill M=2048 (sampled tokens)")
    sample = np.unique(np.r_[0, 2047, np.random.default_rng(5).choice(2048, 10, replace=False)])
    check(sh, synth.CFG_14B, 0, 2048, sample=sample)


def _odd_offset(shape):
    """A bf16 buffer view starting at element 1 of its allocation (2-byte aligned only)."""
    n = int(np.prod(shape))
    big = torch.zeros(n + 16, dtype=torch.int16, device="cuda")
    return big, big[1:1 + n].view(shape)


@pytest.mark.parametrize("M", [2, 40])
def test_outputs_at_odd_element_offsets_match_aligned_ones(M):
    """Outputs that are only element-aligned (the ABI's promise) get the same bits as aligned
    ones: the epilogues fall back from vector stores by address, for the rotary QKV and a
    plain projection, in decode and prefill."""
    sh = SMALL
    w, lb = weights(sh, synth.CFG_TEST, 6)
    x = synth.gen_x(synth.CFG_TEST, 6, 0, M, sh.K)
    pos = synth.gen_positions(synth.CFG_TEST, 6, M, MAX_POS)
    tab = synth.gen_rope_table(MAX_POS, sh.rot, sh.base)
    ref = run(sh, x, w, lb, pos, tab, f32=False)
    bufs = [_odd_offset((M, n, sh.head_dim)) for n in (sh.n_q, sh.n_kv, sh.n_kv)]
    q, k, v = (b[1] for b in bufs)
    qmm.qmm_fused_qkv_rope(dev(x), dev(w.codes), dev(w.scales), dev(w.biases), q, k, v,
                           dev(np.asarray(pos, np.int32)), dev(tab), sh.rot, lin_bias=dev(lb))
    torch.cuda.synchronize()
    say(f"[epilogue] odd-offset outputs, M={M}")
    for got, want in zip((q, k, v), (ref[0], ref[2], ref[3])):
        assert np.array_equal(got.cpu().numpy().view(np.uint16), want)
    for big, _ in bufs:
        assert int(big[0].item()) == 0 and not torch.any(big[1 + big.numel() - 16:] != 0)
    # a plain projection
    lw = synth.gen_weight(synth.CFG_TEST, 7, synth.PROJ_LINEAR, 200, sh.K)
    ya = Guarded((M, 200), False)
    qmm.qmm_linear(dev(x), dev(lw.codes), dev(lw.scales), dev(lw.biases), ya.t)
    big, yo = _odd_offset((M, 200))
    qmm.qmm_linear(dev(x), dev(lw.codes), dev(lw.scales), dev(lw.biases), yo)
    torch.cuda.synchronize()
    assert np.array_equal(yo.cpu().numpy().view(np.uint16), ya.values())
    assert int(big[0].item()) == 0 and not torch.any(big[1 + M * 200:] != 0)


@pytest.mark.parametrize("sh", [SMALL, SMALL_GATED], ids=["full", "gated"])
def test_rope_two_rows_equal_single_row_calls(sh):
    """M = 2 (K <= 5120) runs both rows in one launch of the GEMV, each with its own
    position: the oracle within tolerance, and each row equal to its own M = 1 call bit
    for bit."""
    check(sh, synth.CFG_TEST, 23, 2, contiguous=False)
    w, lb = weights(sh, synth.CFG_TEST, 23)
    x = synth.gen_x(synth.CFG_TEST, 23, 0, 2, sh.K)
    pos = synth.gen_positions(synth.CFG_TEST, 23, 2, MAX_POS, False)
    tab = synth.gen_rope_table(MAX_POS, sh.rot, sh.base)
    both = run(sh, x, w, lb, pos, tab)
    for m in range(2):
        one = run(sh, x[m:m + 1], w, lb, pos[m:m + 1], tab)
        for a, b in zip(both, one):
            if a is not None:
                assert np.array_equal(a[m], b[0]), f"row {m}"
