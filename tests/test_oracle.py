"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: the bf16
field definition and torch's bf16 cast, the packing definition written in the
forward direction, pure-Python brute force with exactly rounded sums, closed
forms for constant codes, the row-concatenation identity of the fusions, the
SwiGLU special values and its derivative bound, and the storage figures the
pages print.  Each is chosen so that a plausible slip in the oracle (a dropped
bias term, a wrong nibble order or group index, a transposed operand, Q/K/V
offsets off by one block, a sign error in the activation) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import qmm_oracle as orc
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bf16_bits(rng, shape, lo_exp=-8, hi_exp=3):
    """Random finite bf16 patterns built from fields (sign, exponent, fraction)."""
    sign = rng.integers(0, 2, size=shape)
    exp = rng.integers(127 + lo_exp, 127 + hi_exp, size=shape)
    frac = rng.integers(0, 128, size=shape)
    return ((sign << 15) | (exp << 7) | frac).astype(np.uint16)


# ---- formats -----------------------------------------------------------------

def test_bf16_decode_every_pattern_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_decode_matches_field_definition():
    for bits in list(range(0, 65536, 97)) + [0x0001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x4300, 0x7F7F, 0xFF7F]:
        v = brute.bf16_value(bits)
        o = float(orc.bf16_to_f64(np.array([bits], np.uint16))[0])
        if math.isnan(v):
            assert math.isnan(o)
        else:
            assert o == v, hex(bits)
    # a few values built from fields
    assert brute.bf16_value(brute.bf16_bits(0, 127, 0)) == 1.0
    assert brute.bf16_value(brute.bf16_bits(1, 128, 64)) == -3.0
    assert brute.bf16_value(brute.bf16_bits(0, 134, 5)) == 133.0


def test_generator_bf16_rounding_is_round_to_nearest_even():
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20], np.float32)
    got = orc.bf16_to_f64(synth.to_bf16_bits(vals))
    assert list(got) == [1.0, 1 + 2 ** -6, 1.0, -1.0, 1 + 2 ** -7]


def test_unpack_inverts_the_packing_definition():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(5, 64))
    words = np.array([brute.pack_row(r) for r in q], dtype=np.uint32)
    assert np.array_equal(orc.unpack_u4(words), q)
    # code 8w+j is nibble j of word w, least significant first
    assert orc.unpack_u4(np.array([[0x87654321]], np.uint32)).tolist() == [[1, 2, 3, 4, 5, 6, 7, 8]]


def test_one_hot_code_lands_on_its_row_and_input():
    N, K = 3, 128
    for n, k in [(0, 0), (1, 9), (2, 127), (1, 64)]:
        q = np.zeros((N, K), int)
        q[n, k] = 15
        words = np.array([brute.pack_row(r) for r in q], np.uint32)
        one = brute.bf16_bits(0, 127, 0)
        s = np.full((N, K // 64), one, np.uint16)
        b = np.zeros((N, K // 64), np.uint16)
        x = np.zeros((1, K), np.uint16)
        x[0, k] = one
        y, _ = orc.linear(x, words, s, b)
        expect = np.zeros((1, N))
        expect[0, n] = 15.0
        assert np.array_equal(y, expect)


def test_storage_matches_the_printed_bits_per_weight():
    fig = json.load(open(os.path.join(GOLDEN, "format_figures.json")))["bits_per_weight"]
    rows, K = 16, 4096
    w = synth.gen_weight(synth.CFG_TEST, 0, 0, rows, K)
    bits = 8 * (w.codes.nbytes + w.scales.nbytes + w.biases.nbytes)
    assert w.codes.dtype == np.uint32 and w.scales.dtype == np.uint16 and w.biases.dtype == np.uint16
    assert bits / (rows * K) == fig["u4"]
    assert K // w.scales.shape[1] == fig["group_size"]
    # the oracle dequantizes exactly that layout
    W = orc.dequant(w.codes, w.scales, w.biases)
    assert W.shape == (rows, K)


@pytest.mark.parametrize("fmt", ["u8", "u6", "u4", "u3"])
def test_storage_of_other_widths_matches_the_printed_bits_per_weight(fmt):
    fig = json.load(open(os.path.join(GOLDEN, "format_figures.json")))["bits_per_weight"]
    bits = int(fmt[1:])
    rows, K = 8, 4096
    w = synth.gen_weight(synth.CFG_TEST, 0, 0, rows, K, bits=bits, group=fig["group_size"])
    assert 8 * (w.codes.nbytes + w.scales.nbytes + w.biases.nbytes) / (rows * K) == fig[fmt]
    assert orc.dequant(w.codes, w.scales, w.biases, bits).shape == (rows, K)


def test_group_sizes_span_the_printed_range():
    fig = json.load(open(os.path.join(GOLDEN, "format_figures.json")))["group_sizes"]
    for G in (fig["min"], 64, fig["max"]):
        w = synth.gen_weight(synth.CFG_TEST, 0, 0, 4, 256, group=G)
        assert w.scales.shape == (4, 256 // G)
        W = orc.dequant(w.codes, w.scales, w.biases)
        q = orc.unpack_u4(w.codes)
        s = orc.bf16_to_f64(w.scales)
        b = orc.bf16_to_f64(w.biases)
        # input k uses the scale and bias of group k // G
        for k in (0, G - 1, G, 255):
            assert np.array_equal(W[:, k], s[:, k // G] * q[:, k] + b[:, k // G])


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_bit_stream_unpack_inverts_the_pure_python_packer(bits):
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 2 ** bits, size=(3, 128))
    words = np.array([brute.pack_row_bits(r, bits) for r in q], np.uint32)
    assert words.shape == (3, 128 * bits // 32)
    assert np.array_equal(orc.unpack_bits(words, bits), q)


def test_bit_stream_order_by_hand():
    """Hand-made words: 3-bit code 10 (stream bits 30..32) straddles words 0 and 1; 6-bit
    code 5 (bits 30..35) straddles too; at 4 bits the stream order is the nibble order."""
    q = [0] * 32
    q[10] = 5                                     # 0b101: bits 30 and 32
    assert brute.pack_row_bits(q, 3) == [0x40000000, 0x00000001, 0]
    assert orc.unpack_bits(np.array([[0x40000000, 0x00000001, 0]], np.uint32), 3).tolist() == [q]
    q6 = [0] * 16
    q6[5] = 0b110011                              # bits 30, 31 in word 0; 34, 35 in word 1
    assert orc.unpack_bits(np.array([[0xC0000000, 0x0000000C, 0]], np.uint32), 6).tolist() == [q6]
    rng_words = np.random.default_rng(3).integers(0, 2 ** 32, size=(4, 16), dtype=np.uint32)
    assert np.array_equal(orc.unpack_bits(rng_words, 4), orc.unpack_u4(rng_words))
    assert orc.unpack_bits(np.array([[0x04030201]], np.uint32), 8).tolist() == [[1, 2, 3, 4]]


def test_e4m3_decode_matches_torch_and_hand_values():
    codes = np.arange(256)
    ours = orc.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2          # 0x7F and 0xFF only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0xB8] == -1.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x07] == 7 * 2.0 ** -9        # smallest normal, largest subnormal


def test_e4m3_weights_dequantize_as_scaled_values():
    w = synth.gen_weight(synth.CFG_TEST, 1, 0, 4, 128, bits="e4m3", bias="uniform")
    assert w.codes.shape == (4, 32) and w.bits == 8
    q = orc.unpack_bits(w.codes, 8)
    assert not np.any((q & 0x7F) == 0x7F)                                  # no NaN codes generated
    W = orc.dequant(w.codes, w.scales, w.biases, orc.E4M3)
    s = orc.bf16_to_f64(w.scales)
    b = orc.bf16_to_f64(w.biases)
    v = orc.e4m3_to_f64(q)
    assert np.array_equal(W, np.repeat(s, 64, 1) * v + np.repeat(b, 64, 1))
    # brute force through the value table
    x = _rand_bf16_bits(np.random.default_rng(7), (2, 128), -3, 2)
    y, A, S, B = orc.project(x, w.codes, w.scales, w.biases, bits=orc.E4M3)
    xv = orc.bf16_to_f64(x)
    ref = np.array([[math.fsum(xv[m, k] * W[n, k] for k in range(128)) for n in range(4)] for m in range(2)])
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * A.max())


@pytest.mark.parametrize("bits,G", [(2, 64), (3, 32), (6, 128), (8, 64), (4, 32), (4, 128)])
def test_oracle_matches_brute_force_other_formats(bits, G):
    M, K, N = 2, 256, 5
    rng = np.random.default_rng(10 * bits + G)
    q = rng.integers(0, 2 ** bits, size=(N, K))
    words = np.array([brute.pack_row_bits(r, bits) for r in q], np.uint32)
    s = _rand_bf16_bits(rng, (N, K // G), -10, -4)
    b = _rand_bf16_bits(rng, (N, K // G), -8, -2)
    x = _rand_bf16_bits(rng, (M, K), -3, 2)
    y, A, S, B = orc.project(x, words, s, b, bits=bits)
    yb, Ab = brute.project(x.tolist(), q.tolist(), s.tolist(), b.tolist(), group=G)
    assert np.allclose(y, np.array(yb), rtol=0, atol=1e-12 * np.array(Ab).max())
    assert np.allclose(A, np.array(Ab), rtol=1e-12)


def test_fused_weight_shape_follows_the_printed_formula():
    fig = json.load(open(os.path.join(GOLDEN, "format_figures.json")))
    ex = fig["fused_qkv_weight_shape"]["example"]
    sh = synth.DENSE_14B
    assert (sh.K, sh.q_out, sh.kv_out) == (ex["hidden"], ex["q_out"], ex["kv_out"])
    w = synth.gen_weight(synth.CFG_TEST, 0, 0, sh.qkv_rows, sh.K)
    assert w.codes.shape == (ex["rows"], ex["cols"])
    d = fig["doubled_q"]
    assert synth.DOUBLED_Q.q_out == d["n_heads"] * d["head_dim"] * 2 == d["q_out"]
    assert synth.DOUBLED_Q.kv_out == d["kv_heads"] * d["head_dim"] == d["kv_out"]
    assert synth.DOUBLED_Q.K == d["hidden"]


# ---- brute force ---------------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(1, 64, 1), (2, 128, 3), (3, 192, 8), (1, 128, 17), (2, 64, 8)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_oracle_matches_brute_force(M, K, N, with_bias):
    rng = np.random.default_rng(1000 * M + 10 * K + N + with_bias)
    q = rng.integers(0, 16, size=(N, K))
    words = np.array([brute.pack_row(r) for r in q], np.uint32)
    s = _rand_bf16_bits(rng, (N, K // 64))
    b = _rand_bf16_bits(rng, (N, K // 64))
    x = _rand_bf16_bits(rng, (M, K), -4, 4)
    lb = _rand_bf16_bits(rng, (N,)) if with_bias else None
    y, A, S, B = orc.project(x, words, s, b, lin_bias=lb)
    yb, Ab = brute.project(x.tolist(), q.tolist(), s.tolist(), b.tolist(),
                           lin_bias_bits=None if lb is None else lb.tolist())
    yb, Ab = np.array(yb), np.array(Ab)
    assert np.all(np.abs(y - yb) <= 1e-12 * Ab + 1e-300)
    assert np.allclose(A, Ab, rtol=1e-12, atol=0)


# ---- closed forms --------------------------------------------------------------

@pytest.mark.parametrize("c", [0, 1, 7, 8, 9, 15])
def test_constant_codes_closed_form(c):
    rng = np.random.default_rng(c)
    N, K = 4, 256
    words = np.full((N, K // 8), c * 0x11111111, np.uint32)
    s = _rand_bf16_bits(rng, (N, K // 64))
    b = _rand_bf16_bits(rng, (N, K // 64))
    x = _rand_bf16_bits(rng, (2, K), -3, 3)
    y, _ = orc.linear(x, words, s, b)
    xv = [[brute.bf16_value(v) for v in row] for row in x.tolist()]
    for m in range(2):
        xs = [math.fsum(xv[m][64 * g:64 * g + 64]) for g in range(K // 64)]
        for n in range(N):
            expect = math.fsum((brute.bf16_value(int(s[n, g])) * c + brute.bf16_value(int(b[n, g]))) * xs[g]
                               for g in range(K // 64))
            assert abs(y[m, n] - expect) <= 1e-12 * (abs(expect) + 1e-30) + 1e-13 * sum(abs(t) for t in xv[m])


def test_constant_codes_single_group_scale():
    """All codes c, one scale s and bias b everywhere: y = (s*c + b) * sum(x)."""
    K, c = 512, 11
    one_half = brute.bf16_bits(0, 126, 0)      # 0.5
    minus3 = brute.bf16_bits(1, 128, 64)       # -3.0
    words = np.full((1, K // 8), c * 0x11111111, np.uint32)
    s = np.full((1, K // 64), one_half, np.uint16)
    b = np.full((1, K // 64), minus3, np.uint16)
    x = synth.gen_x(synth.CFG_TEST, 0, 0, 1, K)
    y, _ = orc.linear(x, words, s, b)
    xsum = math.fsum(brute.bf16_value(v) for v in x[0].tolist())
    assert abs(y[0, 0] - (0.5 * c - 3.0) * xsum) <= 1e-12 * abs(xsum) * 2.5 + 1e-12


def test_scale_and_bias_are_not_swapped_or_dropped():
    """codes 0 -> only the bias survives; bias 0 -> only scale*code."""
    K = 128
    x = np.full((1, K), brute.bf16_bits(0, 127, 0), np.uint16)   # all ones
    two = brute.bf16_bits(0, 128, 0)
    three = brute.bf16_bits(0, 128, 64)
    zero_words = np.zeros((1, K // 8), np.uint32)
    y, _ = orc.linear(x, zero_words, np.full((1, 2), two, np.uint16), np.full((1, 2), three, np.uint16))
    assert y[0, 0] == 3.0 * K
    ones_words = np.full((1, K // 8), 0x11111111, np.uint32)
    y, _ = orc.linear(x, ones_words, np.full((1, 2), two, np.uint16), np.zeros((1, 2), np.uint16))
    assert y[0, 0] == 2.0 * K


def test_group_boundaries_are_64_wide():
    """Different scale per group: a code at input 63 uses group 0, at input 64 group 1."""
    K = 192
    one = brute.bf16_bits(0, 127, 0)
    s = np.array([[brute.bf16_bits(0, 127, 0), brute.bf16_bits(0, 128, 0), brute.bf16_bits(0, 129, 0)]], np.uint16)
    b = np.zeros((1, 3), np.uint16)
    for k, expect in [(0, 1.0), (63, 1.0), (64, 2.0), (127, 2.0), (128, 4.0), (191, 4.0)]:
        q = np.zeros(K, int)
        q[k] = 1
        words = np.array([brute.pack_row(q)], np.uint32)
        x = np.zeros((1, K), np.uint16)
        x[0, k] = one
        y, _ = orc.linear(x, words, s, b)
        assert y[0, 0] == expect, k


# ---- fusion identities --------------------------------------------------------

def test_fused_qkv_equals_three_unfused_projections():
    K, q_out, kv_out = 256, 96, 32
    parts = [synth.gen_weight(synth.CFG_TEST, 1, 0, r, K, index=i, bias="uniform")
             for i, r in enumerate([q_out, kv_out, kv_out])]
    fused = synth.U4Weight.concat(parts)
    lb = synth.gen_lin_bias(synth.CFG_TEST, 1, q_out + 2 * kv_out)
    x = synth.gen_x(synth.CFG_TEST, 1, 0, 3, K)
    (q, k, v), (tq, tk, tv) = orc.fused_qkv(x, fused.codes, fused.scales, fused.biases, q_out, kv_out, lb)
    offs = [0, q_out, q_out + kv_out, q_out + 2 * kv_out]
    for i, (got, tol) in enumerate([(q, tq), (k, tk), (v, tv)]):
        ref, A, S, B = orc.project(x, parts[i].codes, parts[i].scales, parts[i].biases, lb[offs[i]:offs[i + 1]])
        assert np.allclose(got, ref, rtol=0, atol=1e-13 * A.max())
        assert np.allclose(tol, 1e-3 * A, rtol=1e-14)


def test_fused_gate_up_equals_swiglu_of_unfused():
    K, I = 192, 40
    gate = synth.gen_weight(synth.CFG_TEST, 2, 1, I, K, index=0, bias="uniform")
    up = synth.gen_weight(synth.CFG_TEST, 2, 1, I, K, index=1, bias="uniform")
    fused = synth.U4Weight.concat([gate, up])
    x = synth.gen_x(synth.CFG_TEST, 2, 0, 2, K)
    h, _ = orc.gate_up_swiglu(x, fused.codes, fused.scales, fused.biases, I)
    g, _ = orc.linear(x, gate.codes, gate.scales, gate.biases)
    u, _ = orc.linear(x, up.codes, up.scales, up.biases)
    ref = np.array([[brute.silu(float(a)) * float(c) for a, c in zip(gr, ur)] for gr, ur in zip(g, u)])
    assert np.allclose(h, ref, rtol=1e-13, atol=1e-300)
    # the activation goes on the gate half: swapping the halves changes the result
    h_swapped = orc.swiglu(u, g)
    assert not np.allclose(h, h_swapped)


# ---- fused QKV with rotary position embedding -------------------------------------

def _rope_fixture(n_q=2, n_kv=1, hd=8, q_gate=False, K=128, seed=3):
    heads, rows = orc.rope_head_rows(n_q, n_kv, hd, q_gate)
    w = synth.gen_weight(synth.CFG_TEST, seed, synth.PROJ_QKV, rows, K, bias="uniform")
    lb = synth.gen_lin_bias(synth.CFG_TEST, seed, rows)
    return w, lb, heads, rows


def _table(angles):
    """cos/sin table fp32 [P, rot] from angles [P, rot/2] (fp64 -> fp32)."""
    a = np.asarray(angles, np.float64)
    return np.concatenate([np.cos(a), np.sin(a)], axis=1).astype(np.float32)


def _heads_of(y, heads, hd, kind):
    return np.stack([y[:, r0:r0 + hd] for k, h, r0 in heads if k == kind], axis=1)


@pytest.mark.parametrize("q_gate", [False, True])
def test_rope_at_angle_zero_is_the_plain_head_split(q_gate):
    """c = 1, s = 0: every output is the fused projection's row, split per head; the gate
    heads are the second head_dim rows of each doubled query head."""
    hd, rot = 8, 8
    w, lb, heads, rows = _rope_fixture(q_gate=q_gate)
    x = synth.gen_x(synth.CFG_TEST, 4, 0, 3, 128)
    tab = _table(np.zeros((5, rot // 2)))
    (q, g, k, v), (tq, tg, tk, tv) = orc.qkv_rope(x, w.codes, w.scales, w.biases, 2, 1, hd, q_gate, rot,
                                                  [0, 4, 2], tab, lb)
    y, t = orc.linear(x, w.codes, w.scales, w.biases, lb)
    stride = hd * (2 if q_gate else 1)
    assert np.array_equal(q[:, 0], y[:, 0:hd]) and np.array_equal(q[:, 1], y[:, stride:stride + hd])
    if q_gate:
        assert np.array_equal(g[:, 0], y[:, hd:2 * hd]) and np.array_equal(g[:, 1], y[:, 3 * hd:4 * hd])
    else:
        assert g is None
    kv0 = 2 * stride
    assert np.array_equal(k[:, 0], y[:, kv0:kv0 + hd]) and np.array_equal(v[:, 0], y[:, kv0 + hd:kv0 + 2 * hd])
    # the tolerance is the projection's plus only the rotation's fp32 evaluation term
    ya, yb = np.abs(y[:, 0:hd // 2]), np.abs(y[:, hd // 2:hd])
    extra = tq[:, 0] - t[:, 0:hd]
    assert np.all(extra >= 0) and np.all(extra <= 2.0 ** -20 * np.c_[ya + yb, ya + yb])


def test_rope_gate_rows_hold_the_gate():
    """A doubled query head whose gate rows are all zero (codes, scales and biases) gives a
    gate output equal to its additive bias exactly, and queries that are not."""
    hd, rot, K = 8, 8, 64
    w, lb, heads, rows = _rope_fixture(n_q=1, n_kv=1, hd=hd, q_gate=True, K=K)
    c, s_, b = w.codes.copy(), w.scales.copy(), w.biases.copy()
    c[hd:2 * hd] = 0
    s_[hd:2 * hd] = 0
    b[hd:2 * hd] = 0
    x = synth.gen_x(synth.CFG_TEST, 5, 0, 2, K)
    (q, g, k, v), _ = orc.qkv_rope(x, c, s_, b, 1, 1, hd, True, rot, [1, 3], _table(np.full((4, rot // 2), 0.7)), lb)
    assert np.array_equal(g[:, 0], np.broadcast_to(orc.bf16_to_f64(lb[hd:2 * hd]), (2, hd)))
    assert not np.allclose(q[:, 0], orc.bf16_to_f64(lb[0:hd]))


def test_rope_quarter_turn_swaps_the_halves_with_a_sign():
    """c = 0, s = 1 (a quarter turn): rotated dims (a, b) become (-b, a) exactly, in Q and K
    only; dims past rot and all of V pass through."""
    hd, rot = 8, 4
    w, lb, heads, rows = _rope_fixture(hd=hd)
    x = synth.gen_x(synth.CFG_TEST, 6, 0, 2, 128)
    tab = _table(np.full((3, rot // 2), np.pi / 2))
    tab[:, :rot // 2] = 0.0          # cos exactly 0, sin exactly 1
    tab[:, rot // 2:] = 1.0
    (q, g, k, v), _ = orc.qkv_rope(x, w.codes, w.scales, w.biases, 2, 1, hd, False, rot, [2, 1], tab, lb)
    y, _ = orc.linear(x, w.codes, w.scales, w.biases, lb)
    for kind, out in (("q", q), ("k", k)):
        ref = _heads_of(y, heads, hd, kind)
        assert np.array_equal(out[..., 0:2], -ref[..., 2:4])
        assert np.array_equal(out[..., 2:4], ref[..., 0:2])
        assert np.array_equal(out[..., 4:], ref[..., 4:])
    assert np.array_equal(v, _heads_of(y, heads, hd, "v"))


def test_rope_is_complex_multiplication_by_the_position_phase():
    """Half-split rotation = multiplying z_i = d_i + j d_{i+rot/2} by exp(j theta_{p,i}), with
    theta_{p,i} = p * w_i per token position: checked with complex arithmetic and, for
    each pair, the preserved modulus; a token at position p1 + p2 equals the token at p1
    turned by p2 (the phase adds)."""
    hd, rot, P = 16, 12, 40
    w, lb, heads, rows = _rope_fixture(hd=hd, K=192, seed=4)
    omega = 10000.0 ** (-np.arange(rot // 2) * 2.0 / rot)
    ang = np.arange(P)[:, None] * omega[None, :]
    tab = _table(ang)
    x = synth.gen_x(synth.CFG_TEST, 7, 0, 3, 192)
    x = np.concatenate([x[:1], x[:1], x[1:]])   # token 0 twice: positions 7 and 7 + 25
    pos = np.array([7, 32, 3, 39])
    (q, g, k, v), _ = orc.qkv_rope(x, w.codes, w.scales, w.biases, 2, 1, hd, False, rot, pos, tab, lb)
    y, _ = orc.linear(x, w.codes, w.scales, w.biases, lb)
    h = rot // 2
    for kind, out in (("q", q), ("k", k)):
        ref = _heads_of(y, heads, hd, kind)
        z = ref[..., :h] + 1j * ref[..., h:rot]
        cs = tab.astype(np.float64)
        phase = (cs[pos, :h] + 1j * cs[pos, h:rot])[:, None, :]
        zr = z * phase
        assert np.allclose(out[..., :h], zr.real, rtol=0, atol=1e-12)
        assert np.allclose(out[..., h:rot], zr.imag, rtol=0, atol=1e-12)
        assert np.allclose(np.abs(out[..., :h] + 1j * out[..., h:rot]), np.abs(z), rtol=1e-6)
        # the same token at 32 = 7 + 25 is the token at 7 turned by 25 positions
        turn = np.exp(1j * 25 * omega)
        assert np.allclose((out[0, :, :h] + 1j * out[0, :, h:rot]) * turn,
                           out[1, :, :h] + 1j * out[1, :, h:rot], rtol=0, atol=1e-5 * np.abs(z).max())


def test_rope_tolerance_covers_perturbed_inputs():
    """Any projection values within their tolerance rotate to within the rotated tolerance."""
    hd, rot = 8, 8
    w, lb, heads, rows = _rope_fixture(hd=hd)
    x = synth.gen_x(synth.CFG_TEST, 8, 0, 2, 128)
    tab = synth.gen_rope_table(64, rot, 1e4)
    pos = [17, 63]
    (q, _, k, _), (tq, _, tk, _) = orc.qkv_rope(x, w.codes, w.scales, w.biases, 2, 1, hd, False, rot, pos, tab, lb)
    y, t = orc.linear(x, w.codes, w.scales, w.biases, lb)
    ref = _heads_of(y, heads, hd, "q")
    tref = _heads_of(t, heads, hd, "q")
    cs = tab.astype(np.float64)[pos]
    rng = np.random.default_rng(0)
    for _ in range(20):
        e = rng.choice([-1.0, 1.0], size=ref.shape) * tref
        yp = ref + e
        a, b = yp[..., :4], yp[..., 4:]
        c, s = cs[:, None, :4], cs[:, None, 4:]
        ra, rb = a * c - b * s, b * c + a * s
        assert np.all(np.abs(ra - q[..., :4]) <= tq[..., :4]) and np.all(np.abs(rb - q[..., 4:]) <= tq[..., 4:])


def test_rope_table_generator():
    """cos^2 + sin^2 = 1 to fp32 rounding, position 0 is the identity, column i turns at
    base^(-2i/rot) radians per position."""
    tab = synth.gen_rope_table(100, 16, 1e6).astype(np.float64)
    assert np.allclose(tab[:, :8] ** 2 + tab[:, 8:] ** 2, 1.0, atol=1e-6)
    assert np.array_equal(tab[0], np.r_[np.ones(8), np.zeros(8)])
    assert np.allclose(np.arctan2(tab[1, 8:], tab[1, :8]), 1e6 ** (-np.arange(8) * 2.0 / 16), rtol=1e-6)


# ---- SwiGLU -------------------------------------------------------------------

def test_silu_special_values_and_library_agreement():
    g = np.concatenate([np.linspace(-800, 800, 4001), [0.0, -0.0, 1e-300, -1e-300]])
    ours = orc.silu(g)
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.all(np.isfinite(ours))
    assert np.allclose(ours, ref, rtol=1e-14, atol=1e-300)
    assert orc.silu(0.0) == 0.0
    assert orc.silu(50.0) == pytest.approx(50.0, rel=1e-20)
    assert abs(orc.silu(-50.0)) < 1e-19
    for v in [-30.0, -2.5, -1e-3, 0.25, 3.0, 40.0]:
        assert float(orc.silu(v)) == pytest.approx(brute.silu(v), rel=1e-15)


def test_silu_lipschitz_constant():
    g = np.linspace(-20, 20, 2_000_001)
    s = orc.sigmoid(g)
    d = s * (1 + g * (1 - s))
    assert np.max(np.abs(d)) <= orc.SILU_LIPSCHITZ
    assert np.max(np.abs(d)) > orc.SILU_LIPSCHITZ - 2e-4


def test_swiglu_tolerance_covers_worst_case_perturbations():
    rng = np.random.default_rng(5)
    g = rng.standard_normal(20000) * 4
    u = rng.standard_normal(20000) * 4
    tg = np.abs(rng.standard_normal(20000)) * 1e-2
    tu = np.abs(rng.standard_normal(20000)) * 1e-2
    tol = orc.swiglu_tol(g, u, tg, tu)
    h = orc.swiglu(g, u)
    for sg in (-1, 1):
        for su in (-1, 1):
            hp = orc.swiglu(g + sg * tg, u + su * tu)
            assert np.all(np.abs(hp - h) <= tol)
    # and it is not vacuous: the bound is within a small factor of the worst case
    worst = np.max([np.abs(orc.swiglu(g + a * tg, u + b * tu) - h) for a in (-1, 1) for b in (-1, 1)], axis=0)
    assert np.median(tol / np.maximum(worst, 1e-300)) < 2.0


def test_closed_form_gate_and_up_give_known_h():
    """Gate codes all cg, up codes all cu, scale 2^-6, bias 0, x all ones: g = 2^-6*cg*K."""
    K, I = 128, 2
    one = brute.bf16_bits(0, 127, 0)
    s_bits = brute.bf16_bits(0, 121, 0)   # 2^-6
    for cg, cu in [(0, 5), (3, 15), (15, 1)]:
        words = np.concatenate([np.full((I, K // 8), cg * 0x11111111, np.uint32),
                                np.full((I, K // 8), cu * 0x11111111, np.uint32)])
        s = np.full((2 * I, K // 64), s_bits, np.uint16)
        b = np.zeros((2 * I, K // 64), np.uint16)
        x = np.full((1, K), one, np.uint16)
        h, _ = orc.gate_up_swiglu(x, words, s, b, I)
        g, u = cg * K / 64.0, cu * K / 64.0
        expect = g / (1 + math.exp(-g)) * u
        assert np.allclose(h, expect, rtol=1e-15)
    assert orc.swiglu(0.0, 123.0) == 0.0


# ---- routed experts ------------------------------------------------------------

def _moe_fixture(E=6, I=64, K=128, topk=3, seed=0):
    experts_gu = [synth.gen_weight(synth.CFG_TEST, seed, synth.PROJ_MOE_GATE_UP, 2 * I, K, index=e, bias="uniform")
                  for e in range(E)]
    experts_d = [synth.gen_weight(synth.CFG_TEST, seed, synth.PROJ_MOE_DOWN, K, I, index=e, bias="uniform")
                 for e in range(E)]
    return synth.U4Weight.stack(experts_gu), synth.U4Weight.stack(experts_d), experts_gu, experts_d


def test_moe_single_expert_reduces_to_dense():
    gu, d, egu, ed = _moe_fixture()
    K, I = 128, 64
    x = synth.gen_x(synth.CFG_TEST, 3, 0, 1, K)[0]
    for e in range(6):
        h, th = orc.moe_gate_up(x, gu.codes, gu.scales, gu.biases, np.array([e]), 2 * I)
        hd, td = orc.gate_up_swiglu(x, egu[e].codes, egu[e].scales, egu[e].biases, I)
        assert np.array_equal(h[0], hd) and np.array_equal(th[0], td)
        hb = synth.to_bf16_bits(hd)[None, :]
        y, t = orc.moe_down_combine(hb, d.codes, d.scales, d.biases, np.array([e]), np.array([1.0], np.float32))
        yd, td = orc.linear(hb[0], ed[e].codes, ed[e].scales, ed[e].biases)
        assert np.array_equal(y, yd) and np.allclose(t, td)


def test_moe_combine_is_weighted_sum_and_order_free():
    gu, d, egu, ed = _moe_fixture()
    K, I = 128, 64
    x = synth.gen_x(synth.CFG_TEST, 4, 0, 1, K)[0]
    ids = np.array([4, 1, 5], np.int32)
    p = np.array([0.5, 0.3, 0.2], np.float32)
    h, _ = orc.moe_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * I)
    hb = synth.to_bf16_bits(h)
    y, t = orc.moe_down_combine(hb, d.codes, d.scales, d.biases, ids, p)
    ref = sum(float(p[k]) * orc.linear(hb[k], ed[e].codes, ed[e].scales, ed[e].biases)[0] for k, e in enumerate(ids))
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-14 * np.abs(ref).max())
    perm = [2, 0, 1]
    y2, _ = orc.moe_down_combine(hb[perm], d.codes, d.scales, d.biases, ids[perm], p[perm])
    assert np.allclose(y, y2, rtol=1e-13, atol=1e-13 * np.abs(y).max())


def test_moe_out_of_range_id_contributes_nothing():
    gu, d, egu, ed = _moe_fixture()
    K, I = 128, 64
    x = synth.gen_x(synth.CFG_TEST, 5, 0, 1, K)[0]
    ids = np.array([2, -1, 6], np.int32)
    h, _ = orc.moe_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * I)
    assert np.all(h[1] == 0) and np.all(h[2] == 0) and np.any(h[0] != 0)
    hb = synth.to_bf16_bits(np.ones((3, I)))
    p = np.array([0.25, 0.5, 0.25], np.float32)
    y, _ = orc.moe_down_combine(hb, d.codes, d.scales, d.biases, ids, p)
    y_only, _ = orc.moe_down_combine(hb[:1], d.codes, d.scales, d.biases, ids[:1], p[:1])
    assert np.array_equal(y, y_only)


def _prefill_routing(M, E, topk, seed, invalid=True):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)
    if invalid:
        ids[1, 0] = -1          # no expert
        ids[M - 1, topk - 1] = E  # no expert (past the grid)
    p = rng.dirichlet(np.ones(topk), size=M).astype(np.float32)
    return ids, p


def test_moe_prefill_matches_per_token_decode():
    """Prefill (grouped by expert over all tokens) == the decode gather run token by token:
    the grouping and scatter back to (token, slot) are pinned by a different path."""
    gu, d, egu, ed = _moe_fixture()
    K, I, M, topk, E = 128, 64, 7, 3, 6
    x = synth.gen_x(synth.CFG_TEST, 7, 0, M, K)
    ids, p = _prefill_routing(M, E, topk, seed=8)
    h, th = orc.moe_prefill_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * I, bf16_weights=False)
    for m in range(M):
        hd, td = orc.moe_gate_up(x[m], gu.codes, gu.scales, gu.biases, ids[m], 2 * I)
        assert np.allclose(h[m], hd, rtol=1e-13, atol=1e-13 * max(1.0, np.abs(hd).max()))
        assert np.allclose(th[m], td, rtol=1e-12)
    assert np.all(h[1, 0] == 0) and np.all(h[M - 1, topk - 1] == 0)
    hb = synth.to_bf16_bits(h)
    y, t = orc.moe_prefill_down_combine(hb, d.codes, d.scales, d.biases, ids, p, bf16_weights=False)
    for m in range(M):
        yd, td = orc.moe_down_combine(hb[m], d.codes, d.scales, d.biases, ids[m], p[m])
        assert np.allclose(y[m], yd, rtol=1e-12, atol=1e-12 * np.abs(yd).max())
        assert np.allclose(t[m], td, rtol=1e-12)


def test_moe_prefill_bf16_weight_term():
    """With bf16_weights the bound grows by exactly the weight-rounding term of each pair."""
    gu, d, egu, ed = _moe_fixture()
    K, I, M, topk, E = 128, 64, 5, 2, 6
    x = synth.gen_x(synth.CFG_TEST, 9, 0, M, K)
    ids, p = _prefill_routing(M, E, topk, seed=10, invalid=False)
    h0, t0 = orc.moe_prefill_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * I, bf16_weights=False)
    h1, t1 = orc.moe_prefill_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * I, bf16_weights=True)
    assert np.array_equal(h0, h1) and np.all(t1 >= t0) and np.any(t1 > t0)
    m, k = 2, 1
    e = ids[m, k]
    _, tg = orc.gate_up_swiglu(x[m], egu[e].codes, egu[e].scales, egu[e].biases, I, bf16_weights=True)
    assert np.allclose(t1[m, k], tg, rtol=1e-12)


# ---- arithmetic properties ---------------------------------------------------

def test_linearity_and_zero_input():
    w = synth.gen_weight(synth.CFG_TEST, 6, 0, 33, 320)
    x = synth.gen_x(synth.CFG_TEST, 6, 0, 2, 320)
    y, _ = orc.linear(x, w.codes, w.scales, w.biases)
    x2 = synth.to_bf16_bits(2.0 * orc.bf16_to_f64(x))
    y2, _ = orc.linear(x2, w.codes, w.scales, w.biases)
    assert np.array_equal(y2, 2.0 * y)
    y0, A0 = orc.linear(np.zeros_like(x), w.codes, w.scales, w.biases)   # (y, tol): both zero
    assert np.all(y0 == 0) and np.all(A0 == 0)


def test_generated_workload_distribution():
    """The seeded recipe: codes uniform on 0..15, scales in [0.001, 0.01], bias = -8*scale."""
    w = synth.gen_weight(synth.CFG_14B, 0, 0, 512, 5120)
    q = orc.unpack_u4(w.codes)
    counts = np.bincount(q.ravel(), minlength=16)
    assert counts.min() > 0.95 * q.size / 16 and counts.max() < 1.05 * q.size / 16
    s = orc.bf16_to_f64(w.scales)
    b = orc.bf16_to_f64(w.biases)
    assert s.min() >= 0.001 * (1 - 2 ** -8) and s.max() <= 0.01 * (1 + 2 ** -8)
    assert np.array_equal(b, -8 * s)
    W = orc.dequant(w.codes, w.scales, w.biases)
    assert np.allclose(W, s.repeat(64, axis=1) * (q - 8))


def test_oracle_bf16_rounding_matches_torch():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, 3.3895e38]])
    ours = orc.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_scale_mass_and_floor():
    """S = sum|x||s| and B = sum|x||b| from their definitions; the derived evaluation floor is
    0.14 of the stated term 1e-3 * sum|x w| on the workloads' weights (bias = -8 * scale,
    codes uniform: A ~ 4 S and B = 8 S), which is why no workload check adds it; on all-zero
    weights with non-zero codes A is 0 and only the floor remains."""
    w = synth.gen_weight(synth.CFG_14B, 0, 0, 64, 5120)
    x = synth.gen_x(synth.CFG_14B, 0, 0, 1, 5120)
    y, A, S, B = orc.project(x, w.codes, w.scales, w.biases)
    xv = np.abs(orc.bf16_to_f64(x[0]))
    s = np.abs(orc.bf16_to_f64(w.scales))
    b = np.abs(orc.bf16_to_f64(w.biases))
    S_def = np.array([sum(xv[k] * s[n, k // 64] for k in range(0, 5120)) for n in range(3)])
    B_def = np.array([sum(xv[k] * b[n, k // 64] for k in range(0, 5120)) for n in range(3)])
    assert np.allclose(S[0, :3], S_def, rtol=1e-12)
    assert np.allclose(B[0, :3], B_def, rtol=1e-12)
    ratio = orc.eval_floor(S, B) / (orc.REL_TOL * A)
    assert 0.12 < np.median(ratio) < 0.16
    _, t_plain = orc.linear(x, w.codes, w.scales, w.biases)
    assert np.array_equal(t_plain, orc.REL_TOL * A)
    # all-zero weights with non-zero codes: the stated rule alone would demand an exact zero
    z = synth.U4Weight(np.full_like(w.codes, 0x88888888), w.scales, w.biases)
    y0, A0, S0, B0 = orc.project(x, z.codes, z.scales, z.biases)
    assert np.all(y0 == 0) and np.all(A0 == 0) and np.all(S0 > 0)
    _, t0 = orc.linear(x, z.codes, z.scales, z.biases, floor=True)
    assert np.array_equal(t0, orc.eval_floor(S0, B0))


def _f32_chunk_eval(xv, q, s, b):
    """The decode design's fp32 evaluation of one row, written out with float32 steps in the
    least favourable rounding grouping (every product added on its own): per chunk of 32
    inputs D = sum x (128 + q) and X = sum x in input order, t = s*(D - 128 X) + b*X, chunk
    terms added in order.  Test helper only (not the oracle, not the GPU code)."""
    f = np.float32
    acc = f(0)
    for c0 in range(0, len(xv), 32):
        D = f(0)
        X = f(0)
        for k in range(c0, c0 + 32):
            D = f(D + f(xv[k]) * f(128 + int(q[k])))
            X = f(X + f(xv[k]))
        d = f(D - f(128) * X)
        g = (c0 // 64)
        acc = f(acc + f(s[g]) * d)
        acc = f(acc + f(b[g]) * X)
    return float(acc)


@pytest.mark.parametrize("case", ["same-sign", "zero-weights", "random"])
def test_eval_floor_bounds_an_fp32_evaluation(case):
    """The floor is an upper bound of the fp32 evaluation error of the per-group scale/bias
    form, on inputs chosen to make the cancellation D - 128 X as large as it gets (all x
    of one sign, constant code 8 so every weight is exactly zero, or random codes)."""
    rng = np.random.default_rng({"same-sign": 1, "zero-weights": 2, "random": 3}[case])
    K = 2048
    mag = np.exp(rng.uniform(-3, 3, K))          # spread magnitudes: partial sums round unevenly
    x = orc.f32_to_bf16_bits((np.abs(rng.standard_normal(K)) + 0.5) * mag)
    xv = orc.bf16_to_f64(x)
    q = np.full(K, 8) if case == "zero-weights" else rng.integers(0, 16, K)
    if case == "same-sign":
        q = rng.integers(12, 16, K)
    s_bits = orc.f32_to_bf16_bits(rng.uniform(0.001, 0.01, K // 64))
    b_bits = orc.f32_to_bf16_bits(-8.0 * orc.bf16_to_f64(s_bits))
    words = np.array([brute.pack_row(q)], np.uint32)
    y, A, S, B = orc.project(x, words, s_bits[None], b_bits[None])
    got = _f32_chunk_eval(xv, q, orc.bf16_to_f64(s_bits), orc.bf16_to_f64(b_bits))
    err = abs(got - y)
    floor = orc.eval_floor(S, B)
    assert err <= floor
    if case == "zero-weights":
        assert y == 0.0 and err > 0.0      # the stated rule alone would reject this


def test_bf16_weight_rounding_term():
    """R = sum |x| |w - bf16(w)|: zero for weights exact in bf16, equal to the definition
    (torch's bf16 cast of each weight) otherwise, and never above 2^-9 * A."""
    w = synth.gen_weight(synth.CFG_TEST, 12, 0, 24, 256, bias="uniform")
    x = synth.gen_x(synth.CFG_TEST, 12, 0, 3, 256)
    y, A, S, B, R = orc.project(x, w.codes, w.scales, w.biases, bf16_weights=True)
    W = orc.dequant(w.codes, w.scales, w.biases)
    Wb = torch.from_numpy(W).to(torch.bfloat16).to(torch.float64).numpy()
    ref = np.abs(orc.bf16_to_f64(x)) @ np.abs(W - Wb).T
    assert np.allclose(R, ref, rtol=1e-12, atol=0)
    assert np.all(R <= 2.0 ** -9 * A) and np.any(R > 0)
    # codes with q - 8 in {-8,-4,-2,-1,0,1,2,4} and bias -8*scale: every weight is exact
    z = synth.gen_weight(synth.CFG_TEST, 13, 0, 8, 128)
    allowed = np.array([0, 4, 6, 7, 8, 9, 10, 12], np.uint32)
    q = allowed[np.random.default_rng(0).integers(0, 8, size=(8, 128))]
    words = np.array([brute.pack_row(r) for r in q], np.uint32)
    _, _, _, _, R0 = orc.project(x[:, :128], words, z.scales, z.biases, bf16_weights=True)
    assert np.all(R0 == 0)
    _, t_dec = orc.linear(x, w.codes, w.scales, w.biases)
    _, t_pre = orc.linear(x, w.codes, w.scales, w.biases, bf16_weights=True)
    assert np.allclose(t_pre - t_dec, R, rtol=1e-12, atol=1e-300)
