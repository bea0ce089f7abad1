"""The prefill GEMM's last partial round: when the tiles fill some whole rounds of one block
per CU and leave a remainder of at most half the CUs, the remainder runs as half-height
blocks (128 rows of x each, two per tile) in a launch of its own.  Shapes here are chosen
from the device's CU count so that the grid is two row tiles x (CUs / 2 + 2) column tiles:
one whole round and 4 tiles left.  Each output row depends on its own activation row only,
so the same rows computed in calls whose grids do not split (the first 256 rows, then the
rest) must give the same bits; the oracle checks the values."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import bf16_term, assert_within, say
from test_gemm_parity import run_gate_up, run_linear, run_qkv
import test_rope_parity as rope

pytestmark = pytest.mark.gpu

M, K = 300, 128  # two row tiles, the second ragged


def col_tiles():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return cus // 2 + 2  # 2 * this = CUs + 4 tiles: one round and 4 left


def test_split_tail_linear():
    N = 256 * col_tiles()
    say(f"[gemm tail] linear M={M} K={K} N={N}")
    w = synth.gen_weight(synth.CFG_TEST, 400, synth.PROJ_LINEAR, N, K)
    x = synth.gen_x(synth.CFG_TEST, 400, 0, M, K)
    y, t = orc.linear(x, w.codes, w.scales, w.biases, bf16_weights=bf16_term(M, K))
    got = run_linear(x, w)
    assert_within(got, y, t, "split-tail linear")
    assert np.array_equal(got, np.concatenate([run_linear(x[:256], w), run_linear(x[256:], w)]))


def test_split_tail_fused_qkv():
    kv_out = 256
    q_out = 256 * col_tiles() - 2 * kv_out  # the tail tiles hold the K and V columns
    say(f"[gemm tail] fused QKV M={M} K={K} q_out={q_out} kv_out={kv_out}")
    w = synth.gen_weight(synth.CFG_TEST, 401, synth.PROJ_QKV, q_out + 2 * kv_out, K, bias="uniform")
    x = synth.gen_x(synth.CFG_TEST, 401, 0, M, K)
    (q, k, v), (tq, tk, tv) = orc.fused_qkv(x, w.codes, w.scales, w.biases, q_out, kv_out,
                                            bf16_weights=bf16_term(M, K))
    got = run_qkv(x, w, q_out, kv_out)
    for g, r, tol, nm in zip(got, (q, k, v), (tq, tk, tv), "QKV"):
        assert_within(g, r, tol, f"split-tail {nm}")
    a, b = run_qkv(x[:256], w, q_out, kv_out), run_qkv(x[256:], w, q_out, kv_out)
    for g, ga, gb in zip(got, a, b):
        assert np.array_equal(g, np.concatenate([ga, gb]))


def test_split_tail_gate_up():
    I = 128 * col_tiles()
    say(f"[gemm tail] gate+up M={M} K={K} I={I}")
    w = synth.gen_weight(synth.CFG_TEST, 402, synth.PROJ_GATE_UP, 2 * I, K)
    x = synth.gen_x(synth.CFG_TEST, 402, 0, M, K)
    h, th = orc.gate_up_swiglu(x, w.codes, w.scales, w.biases, I, bf16_weights=bf16_term(M, K))
    got = run_gate_up(x, w, I)
    assert_within(got, h, th, "split-tail gate+up")
    assert np.array_equal(got, np.concatenate([run_gate_up(x[:256], w, I), run_gate_up(x[256:], w, I)]))


def test_split_tail_qkv_rope():
    heads = 256 * col_tiles() // 128  # rotating pairs fill col_tiles() tiles of 128 pairs
    sh = synth.RopeShape(f"QKV + RoPE (hidden {K}, {heads - 4} q / 2 kv heads x 128, full rotary)",
                         K, heads - 4, 2, 128, False, 128, 1.0e4)
    say(f"[gemm tail] {sh.name} M={M}")
    rope.check(sh, synth.CFG_TEST, 403, M)
