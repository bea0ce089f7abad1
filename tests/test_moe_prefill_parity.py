"""GPU parity of the routed experts over a batch of tokens (prefill) against the fp64
oracle: routing + gathered gate+up+SwiGLU (stage 1), routing + gathered down + combine
(stage 2).  Stage 2 reads an h made by the oracle (or seeded), never the GPU's stage 1.
The gathered GEMM rounds dequantized weights to bf16; the oracle adds that rounding's
bound (bf16_weights) only at short K (`bf16_term`), the stated rule alone otherwise."""
import numpy as np
import pytest
import torch

import gemm_affine_u4_amd as qmm
import synth
from oracle import qmm_oracle as orc
from gpu_util import bf16_term, Guarded, assert_within, dev, rne_bits_of, say

pytestmark = pytest.mark.gpu


class Routed:
    """A routed workspace for (ids, E) sized for a down projection of out_rows rows."""

    def __init__(self, ids: np.ndarray, E: int, out_rows: int):
        M, topk = ids.shape
        n = qmm.qmm_moe_prefill_workspace_bytes(M, topk, E, out_rows)
        assert n > 0
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        self.ids = dev(np.ascontiguousarray(ids, np.int32))
        self.E = E
        qmm.qmm_moe_route(self.ids, E, self.ws)


def stage1(x_bits, grid, r: Routed, I, f32=True):
    M, topk = r.ids.shape
    out = Guarded((M, topk, I), f32)
    qmm.qmm_moe_prefill(qmm.QMM_MOE_GATE_UP_SWIGLU, dev(x_bits), dev(grid.codes), dev(grid.scales),
                        dev(grid.biases), r.ids, r.ws, out.t)
    torch.cuda.synchronize()
    return out.values()


def stage2(h_bits, grid, r: Routed, p, f32=True):
    M, topk = r.ids.shape
    rows = grid.codes.shape[1]
    out = Guarded((M, rows), f32)
    qmm.qmm_moe_prefill(qmm.QMM_MOE_DOWN_COMBINE, dev(h_bits), dev(grid.codes), dev(grid.scales),
                        dev(grid.biases), r.ids, r.ws, out.t, expert_w=dev(np.asarray(p, np.float32)))
    torch.cuda.synchronize()
    return out.values()


def grids(shape: synth.MoEShape, cfg: int, layer: int):
    gu = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_GATE_UP, shape.E, 2 * shape.I, shape.hidden)
    dn = synth.gen_expert_grid(cfg, layer, synth.PROJ_MOE_DOWN, shape.E, shape.hidden, shape.I)
    return gu, dn


def check_both_stages(shape, cfg, layer, M, ids, p, what):
    gu, dn = grids(shape, cfg, layer)
    x = synth.gen_x(cfg, layer, 0, M, shape.hidden)
    r = Routed(ids, shape.E, shape.hidden)
    h, th = orc.moe_prefill_gate_up(x, gu.codes, gu.scales, gu.biases, ids, 2 * shape.I,
                                     bf16_weights=bf16_term(M, shape.hidden))
    g1 = stage1(x, gu, r, shape.I)
    assert_within(g1, h, th, f"{what}: stage 1 h")
    assert np.array_equal(stage1(x, gu, r, shape.I, f32=False), rne_bits_of(g1))
    h_bits = orc.f32_to_bf16_bits(h)   # the oracle's own h, rounded, feeds both sides
    y, ty = orc.moe_prefill_down_combine(h_bits, dn.codes, dn.scales, dn.biases, ids, p,
                                         bf16_weights=bf16_term(M, shape.I))
    g2 = stage2(h_bits, dn, r, p)
    assert_within(g2, y, ty, f"{what}: stage 2 y")
    assert np.array_equal(stage2(h_bits, dn, r, p, f32=False), rne_bits_of(g2))
    return g1, g2


# Several routing tiles per expert (skewed popularity: one expert above 256 pairs, one
# nearly empty), a ragged last tile everywhere, I and hidden not multiples of the tile.
SMALL = synth.MoEShape("small MoE prefill (hidden 320, 8 experts, I 192, top-2)", 320, 8, 192, 2)


def test_moe_prefill_several_tiles_per_expert():
    M = 600
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 0, M, SMALL.E, SMALL.topk, skew=1.0)
    counts = np.bincount(ids.ravel(), minlength=SMALL.E)
    say(f"[moe prefill] {SMALL.name}, M={M}, pairs per expert {counts.tolist()}")
    assert counts.max() > 256 and counts.min() < 256
    check_both_stages(SMALL, synth.CFG_TEST, 0, M, ids, p, "several tiles")


def test_moe_prefill_no_expert_ids_repeats_and_empty_experts():
    shape = synth.MoEShape("small MoE prefill (hidden 256, 6 experts, I 64, top-3)", 256, 6, 64, 3)
    M = 37
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 1, M, 4, shape.topk)   # experts 4, 5 get nothing
    ids[1, 0] = -1
    ids[5, 2] = shape.E        # past the grid: no expert
    ids[9, :] = -7             # a token with no expert at all
    ids[12, 1] = ids[12, 0]    # the same expert twice for one token
    say(f"[moe prefill] ids with no expert, repeats, empty experts (M={M})")
    g1, g2 = check_both_stages(shape, synth.CFG_TEST, 1, M, ids, p, "gaps")
    assert np.all(g1[1, 0] == 0) and np.all(g1[5, 2] == 0) and np.all(g1[9] == 0)
    assert np.array_equal(g1[12, 0], g1[12, 1])
    assert np.all(g2[9] == 0)


@pytest.mark.parametrize("M", [1, 9, 255, 257])
def test_moe_prefill_small_batches(M):
    shape = SMALL
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 2, M, shape.E, shape.topk)
    say(f"[moe prefill] M={M}")
    check_both_stages(shape, synth.CFG_TEST, 2, M, ids, p, f"M={M}")


def test_moe_prefill_is_deterministic_and_workspace_reusable():
    """The same call twice gives the same bits; a workspace routed again for other ids
    (fewer tokens) gives what a fresh workspace gives."""
    shape = SMALL
    gu, dn = grids(shape, synth.CFG_TEST, 3)
    ids_a, p_a = synth.gen_prefill_routing(synth.CFG_TEST, 3, 300, shape.E, shape.topk, skew=1.0)
    ids_b, p_b = synth.gen_prefill_routing(synth.CFG_TEST, 4, 120, shape.E, shape.topk)
    xa = synth.gen_x(synth.CFG_TEST, 3, 0, 300, shape.hidden)
    xb = synth.gen_x(synth.CFG_TEST, 3, 1, 120, shape.hidden)
    ra = Routed(ids_a, shape.E, shape.hidden)
    a1 = stage1(xa, gu, ra, shape.I)
    assert np.array_equal(a1, stage1(xa, gu, ra, shape.I))
    hb = synth.gen_x(synth.CFG_TEST, 3, 2, 300 * shape.topk, shape.I).reshape(300, shape.topk, shape.I)
    a2 = stage2(hb, dn, ra, p_a)
    assert np.array_equal(a2, stage2(hb, dn, ra, p_a))
    # reuse ra's workspace for ids_b
    rb = Routed.__new__(Routed)
    rb.ws, rb.E = ra.ws, shape.E
    rb.ids = dev(ids_b)
    qmm.qmm_moe_route(rb.ids, shape.E, rb.ws)
    fresh = Routed(ids_b, shape.E, shape.hidden)
    b1 = stage1(xb, gu, rb, shape.I)
    assert np.array_equal(b1, stage1(xb, gu, fresh, shape.I))
    hbb = synth.gen_x(synth.CFG_TEST, 3, 3, 120 * shape.topk, shape.I).reshape(120, shape.topk, shape.I)
    assert np.array_equal(stage2(hbb, dn, rb, p_b), stage2(hbb, dn, fresh, p_b))


def test_moe_prefill_35B_shape_full_batch_sampled_tokens():
    """The 35B-A3B-shaped workload at its full batch (2048 tokens, top-8 of 256 experts),
    in the launch configuration the bench times; the oracle checks a sample of tokens
    (each token's outputs depend on that token's inputs and experts only)."""
    shape = synth.MOE_35B
    M = synth.MOE_PREFILL_M
    cfg = synth.CFG_MOE
    gu, dn = grids(shape, cfg, 0)
    ids, p = synth.gen_prefill_routing(cfg, 0, M, shape.E, shape.topk)
    x = synth.gen_x(cfg, 0, 0, M, shape.hidden)
    # stage-2 input: seeded bf16 h of the magnitude SwiGLU outputs have here
    h_in = synth.to_bf16_bits(0.05 * synth.bf16_bits_to_f32(synth.gen_x(cfg, 0, 1, M * shape.topk, shape.I)))
    h_in = h_in.reshape(M, shape.topk, shape.I)
    say(f"[moe prefill] {shape.name}, M={M}")
    r = Routed(ids, shape.E, shape.hidden)
    g1 = stage1(x, gu, r, shape.I)
    g2 = stage2(h_in, dn, r, p)
    sample = np.unique(np.r_[0, M - 1, np.random.default_rng(11).choice(M, 14, replace=False)])
    h, th = orc.moe_prefill_gate_up(x[sample], gu.codes, gu.scales, gu.biases, ids[sample], 2 * shape.I,
                                     bf16_weights=bf16_term(M, shape.hidden))
    assert_within(g1[sample], h, th, "35B stage 1 (sampled tokens)")
    y, ty = orc.moe_prefill_down_combine(h_in[sample], dn.codes, dn.scales, dn.biases, ids[sample], p[sample],
                                         bf16_weights=bf16_term(M, shape.I))
    assert_within(g2[sample], y, ty, "35B stage 2 (sampled tokens)")


def test_small_batch_pair_path_and_wide_expert():
    """Few pairs (M * topk <= 288) run the decode gather kernels pair by pair and the
    routing call does nothing; a down projection wider than those kernels take (expert
    I = 5632 > 5120) makes stage 2 route on its own and run the routed kernel."""
    shape = synth.MoEShape("wide-expert MoE (hidden 128, 4 experts, I 5632, top-2)", 128, 4, 5632, 2)
    M = 5
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 7, M, shape.E, shape.topk)
    say(f"[moe prefill] {shape.name}, M={M}")
    check_both_stages(shape, synth.CFG_TEST, 7, M, ids, p, "wide expert")


def test_moe_prefill_one_hot_expert_among_small_ones():
    """1200 pairs over 64 experts: one expert takes slot 0 of 300 tokens (three routing
    tiles of up to 128 pairs, the last ragged), the others a few pairs each (one ragged
    32-pair block), one pair has no expert; K = 1024 and K = 512."""
    shape = synth.MoEShape("MoE prefill (hidden 1024, 64 experts, I 512, top-3)", 1024, 64, 512, 3)
    M = 400
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 8, M, shape.E, shape.topk)
    ids[:300, 0] = 5
    ids[7, 2] = -1
    counts = np.bincount(ids[ids >= 0].ravel(), minlength=shape.E)
    say(f"[moe prefill] {shape.name}, M={M}, pairs per expert max {counts.max()} min {counts.min()}")
    assert counts.max() > 256
    g1, _ = check_both_stages(shape, synth.CFG_TEST, 8, M, ids, p, "one hot expert")
    assert np.all(g1[7, 2] == 0)


def test_moe_prefill_hidden_1024_37_pairs_per_expert():
    """1200 pairs over 32 experts (about 37 each: tiles of one or two 32-pair blocks),
    hidden 1024 (16 K steps, two scale chunks per row) and I = 512."""
    shape = synth.MoEShape("MoE prefill (hidden 1024, 32 experts, I 512, top-3)", 1024, 32, 512, 3)
    M = 400
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 9, M, shape.E, shape.topk)
    say(f"[moe prefill] {shape.name}, M={M}")
    check_both_stages(shape, synth.CFG_TEST, 9, M, ids, p, "hidden 1024")


def test_moe_prefill_routed_shortest_k():
    """The routed kernel at its shortest K: stage 1 at K = 128 (two steps, one code chunk)
    and stage 2 at K = 64 (one step), 600 pairs over 6 experts, one pair without an
    expert."""
    shape = synth.MoEShape("MoE prefill (hidden 128, 6 experts, I 64, top-2)", 128, 6, 64, 2)
    M = 300
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 12, M, shape.E, shape.topk, skew=1.0)
    ids[3, 1] = -1
    assert M * shape.topk > 288
    say(f"[moe prefill] {shape.name}, M={M}")
    g1, _ = check_both_stages(shape, synth.CFG_TEST, 12, M, ids, p, "shortest K")
    assert np.all(g1[3, 1] == 0)


def test_moe_prefill_many_chunks_and_ragged_expert_count():
    """4800 pairs (19 routing chunks: the scan's wave-per-expert path) over 100 experts
    (not a multiple of the scan's batch of 8), skewed, some experts empty."""
    shape = synth.MoEShape("MoE prefill (hidden 320, 100 experts, I 192, top-4)", 320, 100, 192, 4)
    M = 1200
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 10, M, 90, shape.topk, skew=1.0)  # experts 90.. empty
    say(f"[moe prefill] {shape.name}, M={M}")
    check_both_stages(shape, synth.CFG_TEST, 10, M, ids, p, "many chunks")


def test_moe_prefill_long_k():
    """Stage 1 at K = 6144 (96 K steps, 12 scale chunks per row): 600 pairs over 32
    experts, skewed."""
    shape = synth.MoEShape("MoE prefill (hidden 6144, 32 experts, I 512, top-2)", 6144, 32, 512, 2)
    M = 300
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 11, M, shape.E, shape.topk, skew=1.0)
    assert 288 < M * shape.topk
    say(f"[moe prefill] {shape.name}, M={M}")
    check_both_stages(shape, synth.CFG_TEST, 11, M, ids, p, "long K")


def test_moe_prefill_35B_shape_128_tokens():
    """The 35B-A3B shape at 128 tokens (1024 pairs over 256 experts, about 4 each: tiles of
    one 32-pair block), routed (K = 2048 and K = 512)."""
    shape = synth.MOE_35B
    M = 128
    ids, p = synth.gen_prefill_routing(synth.CFG_MOE, 1, M, shape.E, shape.topk)
    say(f"[moe prefill] {shape.name}, M={M}")
    check_both_stages(shape, synth.CFG_MOE, 1, M, ids, p, "35B M=128")


def test_moe_prefill_1500_experts():
    """1500 experts (hidden 128, I 64, top-2, 400 tokens: most experts get no pair, none
    more than a few): above 1024 experts the routing runs as three kernels even for few
    pairs; a pair with no expert."""
    shape = synth.MoEShape("MoE prefill (hidden 128, 1500 experts, I 64, top-2)", 128, 1500, 64, 2)
    M = 400
    ids, p = synth.gen_prefill_routing(synth.CFG_TEST, 10, M, shape.E, shape.topk, skew=1.0)
    ids[3, 1] = -1
    say(f"[moe prefill] {shape.name}, M={M}, experts used {len(np.unique(ids[ids >= 0]))}")
    g1, _ = check_both_stages(shape, synth.CFG_TEST, 10, M, ids, p, "1500 experts")
    assert np.all(g1[3, 1] == 0)


def test_moe_prefill_routing_above_16384_pairs():
    """Above 16384 (token, slot) pairs the routing runs as three kernels (bucket positions
    in pair order) instead of one block (positions in the order its atomics took): 8256
    tokens x top-8 of 64 experts (hidden 128, I 64), ~1000 pairs per expert.  The oracle
    checks a sample of tokens of both stages; the first 2048 tokens alone (16384 pairs, one
    block) give the same bits for those tokens, since a pair's outputs do not depend on
    where it sits in its expert's tiles."""
    shape = synth.MoEShape("MoE prefill (hidden 128, 64 experts, I 64, top-8)", 128, 64, 64, 8)
    M, Ms = 8256, 2048
    cfg = synth.CFG_TEST
    ids, p = synth.gen_prefill_routing(cfg, 12, M, shape.E, shape.topk)
    ids[100, 5] = -1
    assert M * shape.topk > 16384 and Ms * shape.topk == 16384
    gu, dn = grids(shape, cfg, 12)
    x = synth.gen_x(cfg, 12, 0, M, shape.hidden)
    h_in = synth.to_bf16_bits(0.05 * synth.bf16_bits_to_f32(synth.gen_x(cfg, 12, 1, M * shape.topk, shape.I)))
    h_in = h_in.reshape(M, shape.topk, shape.I)
    say(f"[moe prefill] {shape.name}, M={M} and its first {Ms} tokens")
    r = Routed(ids, shape.E, shape.hidden)
    g1 = stage1(x, gu, r, shape.I)
    g2 = stage2(h_in, dn, r, p)
    assert np.all(g1[100, 5] == 0)
    sample = np.unique(np.r_[0, 100, M - 1, np.random.default_rng(12).choice(M, 13, replace=False)])
    h, th = orc.moe_prefill_gate_up(x[sample], gu.codes, gu.scales, gu.biases, ids[sample], 2 * shape.I,
                                     bf16_weights=bf16_term(M, shape.hidden))
    assert_within(g1[sample], h, th, "16384+ pairs, stage 1 (sampled tokens)")
    y, ty = orc.moe_prefill_down_combine(h_in[sample], dn.codes, dn.scales, dn.biases, ids[sample], p[sample],
                                         bf16_weights=bf16_term(M, shape.I))
    assert_within(g2[sample], y, ty, "16384+ pairs, stage 2 (sampled tokens)")
    rs = Routed(ids[:Ms], shape.E, shape.hidden)
    assert np.array_equal(stage1(x[:Ms], gu, rs, shape.I), g1[:Ms])
    assert np.array_equal(stage2(h_in[:Ms], dn, rs, p[:Ms]), g2[:Ms])
