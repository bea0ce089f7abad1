"""Seeded synthetic inputs for the u4 group-64 affine quantized matmul.

This module only draws random numbers and stores them in the formats the
library takes as input (uint32 words of packed 4-bit codes, bf16 bit
patterns, int32 expert ids, fp32 combine weights).  It holds none of the
method's arithmetic: it never unpacks a code, never dequantizes and never
forms a product.  Both the CPU oracle and the GPU path read their inputs
from here, so it is the one piece of Python they share.

Distributions (the workloads of the five decode/prefill shapes):
  * codes: every 4-bit code uniform on 0..15, independently.  A uint32 drawn
    uniformly on [0, 2**32) has exactly that distribution in each of its eight
    nibbles, so words are drawn directly and no packing is performed here.
  * scales: fp32 uniform on [0.001, 0.01], rounded to bf16 (round to nearest
    even, done by torch's float32 -> bfloat16 cast).
  * biases: bf16(-8 * scale), which is exact (a power-of-two multiple), so that
    the dequantized weight is scale * (code - 8).
  * activations: fp32 standard normal, rounded to bf16.
  * MoE routing: distinct expert ids drawn uniformly without replacement, and
    combine weights softmax(N(0,1) logits) computed in fp64 and cast to fp32.
    The router is upstream of the quantized matmul; its output is an input.

Every stream is seeded by numpy SeedSequence([cfg, layer, proj, field, index]).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# proj ids
PROJ_QKV, PROJ_GATE_UP, PROJ_DOWN, PROJ_MOE_GATE_UP, PROJ_MOE_DOWN, PROJ_LINEAR = 0, 1, 2, 3, 4, 5
# field ids
F_CODES, F_SCALES, F_X, F_IDS, F_LOGITS, F_LINBIAS, F_BIASES = 0, 1, 2, 3, 4, 5, 6

GROUP = 64          # inputs per scale/bias group
CODES_PER_WORD = 8  # 4-bit codes per uint32


def rng(cfg: int, layer: int, proj: int, field: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg, layer, proj, field, index]))


def to_bf16_bits(a) -> np.ndarray:
    """fp32/fp64 array -> bf16 bit patterns (uint16), round to nearest even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values via torch's bf16 -> fp32 cast (input plumbing only)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


@dataclass
class U4Weight:
    """Packed weight of `rows` output rows over `K` inputs (host arrays)."""
    codes: np.ndarray   # uint32 [rows, K*bits/32]
    scales: np.ndarray  # uint16 bf16 bits [rows, K/group]
    biases: np.ndarray  # uint16 bf16 bits [rows, K/group]
    bits: int = 4

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def K(self) -> int:
        return self.codes.shape[-1] * 32 // self.bits

    def slice_rows(self, r0: int, r1: int) -> "U4Weight":
        return U4Weight(self.codes[r0:r1], self.scales[r0:r1], self.biases[r0:r1], self.bits)

    def take_rows(self, idx) -> "U4Weight":
        idx = np.asarray(idx)
        return U4Weight(self.codes[idx], self.scales[idx], self.biases[idx], self.bits)

    @staticmethod
    def concat(parts) -> "U4Weight":
        return U4Weight(np.concatenate([p.codes for p in parts]),
                        np.concatenate([p.scales for p in parts]),
                        np.concatenate([p.biases for p in parts]), parts[0].bits)

    @staticmethod
    def stack(parts) -> "U4Weight":
        return U4Weight(np.stack([p.codes for p in parts]),
                        np.stack([p.scales for p in parts]),
                        np.stack([p.biases for p in parts]), parts[0].bits)


def gen_weight(cfg: int, layer: int, proj: int, rows: int, K: int, index: int = 0,
               scale_lo: float = 0.001, scale_hi: float = 0.01, bias: str = "minus8",
               bits: int = 4, group: int = GROUP) -> U4Weight:
    """Seeded packed weight: codes uint32 [rows, K*bits/32] (uniform random words, so every
    code is uniform on 0 .. 2^bits - 1), bf16 scales and biases [rows, K/group].
    bias='minus8' centres the codes: bias = -2^(bits-1) * scale (-8 * scale at 4 bits, the
    workloads' recipe); bias='uniform' draws an independent bias uniform on
    [-scale_hi*8, scale_hi*8] (tests only)."""
    if K % 64 or K % group:
        raise ValueError("K must be a multiple of 64 and of the group size")
    if bits == "e4m3":
        # fp8 e4m3 codes: uniform over the 254 finite patterns (0x7F and 0xFF are NaN),
        # signed values, so no centring bias
        b8 = rng(cfg, layer, proj, F_CODES, index).integers(0, 254, size=(rows, K), dtype=np.int64)
        b8 = np.where(b8 >= 0x7F, b8 + 1, b8).astype(np.uint8)
        codes = np.ascontiguousarray(b8).view("<u4").astype(np.uint32)
        s32 = rng(cfg, layer, proj, F_SCALES, index).uniform(scale_lo, scale_hi, size=(rows, K // group)).astype(np.float32)
        scales = to_bf16_bits(s32)
        if bias == "uniform":
            b = rng(cfg, layer, proj, F_BIASES, index).uniform(-8 * scale_hi, 8 * scale_hi, size=(rows, K // group))
            biases = to_bf16_bits(b)
        else:
            biases = np.zeros_like(scales)
        return U4Weight(codes, scales, biases, 8)
    codes = rng(cfg, layer, proj, F_CODES, index).integers(0, 2 ** 32, size=(rows, K * bits // 32),
                                                          dtype=np.uint32)
    s32 = rng(cfg, layer, proj, F_SCALES, index).uniform(scale_lo, scale_hi, size=(rows, K // group)).astype(np.float32)
    scales = to_bf16_bits(s32)
    if bias == "minus8":
        biases = to_bf16_bits(-float(2 ** (bits - 1)) * bf16_bits_to_f32(scales))
    elif bias == "uniform":
        b = rng(cfg, layer, proj, F_BIASES, index).uniform(-8 * scale_hi, 8 * scale_hi, size=(rows, K // group))
        biases = to_bf16_bits(b)
    else:
        raise ValueError(bias)
    return U4Weight(codes, scales, biases, bits)


def gen_x(cfg: int, layer: int, step: int, M: int, K: int, magnitude: str = "normal") -> np.ndarray:
    """Seeded activations as bf16 bits [M, K]. magnitude='varied' multiplies each element
    by 10**U(-3, 3) (the varied-magnitude projection case)."""
    g = rng(cfg, layer, 0, F_X, step)
    x = g.standard_normal(size=(M, K), dtype=np.float32)
    if magnitude == "varied":
        x = x * (10.0 ** g.uniform(-3.0, 3.0, size=(M, K))).astype(np.float32)
    elif magnitude != "normal":
        raise ValueError(magnitude)
    return to_bf16_bits(x)


def gen_lin_bias(cfg: int, layer: int, rows: int) -> np.ndarray:
    """Seeded optional additive output bias (bf16 bits [rows]) for the QKV path."""
    return to_bf16_bits(rng(cfg, layer, PROJ_QKV, F_LINBIAS).standard_normal(rows).astype(np.float32))


def gen_routing(cfg: int, layer: int, step: int, E: int, topk: int):
    """topk distinct expert ids uniform over [0, E) and fp32 softmax(N(0,1)) combine weights."""
    ids = rng(cfg, layer, PROJ_MOE_GATE_UP, F_IDS, step).choice(E, size=topk, replace=False).astype(np.int32)
    logits = rng(cfg, layer, PROJ_MOE_GATE_UP, F_LOGITS, step).standard_normal(topk)
    e = np.exp(logits - logits.max())
    p = (e / e.sum()).astype(np.float32)
    return ids, p


def gen_prefill_routing(cfg: int, layer: int, M: int, E: int, topk: int, skew: float = 0.5):
    """Routing of M tokens: each token takes topk distinct experts, drawn without
    replacement in proportion to a seeded per-expert popularity exp(skew * N(0,1)) (so
    some experts get many more tokens than others, as a trained router's do), and fp32
    softmax(N(0,1)) combine weights.  Returns (ids int32 [M, topk], p fp32 [M, topk])."""
    pop = skew * rng(cfg, layer, PROJ_MOE_GATE_UP, F_IDS, 1 << 20).standard_normal(E)
    # Gumbel top-k: the topk largest of log-popularity + Gumbel noise are a draw
    # without replacement proportional to the popularity.
    g = rng(cfg, layer, PROJ_MOE_GATE_UP, F_IDS, (1 << 20) + 1).gumbel(size=(M, E))
    ids = np.argsort(-(pop[None, :] + g), axis=1, kind="stable")[:, :topk].astype(np.int32)
    logits = rng(cfg, layer, PROJ_MOE_GATE_UP, F_LOGITS, 1 << 20).standard_normal((M, topk))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, p


def gen_rope_table(max_pos: int, rot: int, base: float = 1.0e6) -> np.ndarray:
    """Rotary table fp32 [max_pos, rot]: cos in [:, :rot/2], sin in [:, rot/2:], at the
    angle fp32(p) * inv_freq_i with inv_freq_i = fp32(base^(-2i/rot)) rounded to fp32
    (the usual construction), cos/sin of that fp32 angle rounded to fp32."""
    half = rot // 2
    inv = (base ** (-(2.0 * np.arange(half)) / rot)).astype(np.float32)
    ang = (np.arange(max_pos, dtype=np.float32)[:, None] * inv[None, :]).astype(np.float32)
    a64 = ang.astype(np.float64)
    return np.concatenate([np.cos(a64), np.sin(a64)], axis=1).astype(np.float32)


def gen_positions(cfg: int, layer: int, M: int, max_pos: int, contiguous: bool = True) -> np.ndarray:
    """int32 positions of M tokens: a seeded start and M consecutive positions (a prompt
    chunk), or M independent positions (tokens of different sequences)."""
    g = rng(cfg, layer, PROJ_QKV, F_IDS, 1 << 21)
    if contiguous:
        start = int(g.integers(0, max(1, max_pos - M + 1)))
        return np.arange(start, start + M, dtype=np.int32)
    return g.integers(0, max_pos, size=M).astype(np.int32)


def gen_expert_grid(cfg: int, layer: int, proj: int, E: int, rows: int, K: int,
                    experts=None, bits: int = 4, group: int = GROUP) -> U4Weight:
    """3-D expert grid [E, rows, ...]; expert e is seeded by index=e, so any subset of
    experts can be regenerated on its own.  `experts` limits generation to a subset
    (the others are left zero), for oracle-side regeneration."""
    codes = np.zeros((E, rows, K * (8 if bits == "e4m3" else bits) // 32), np.uint32)
    scales = np.zeros((E, rows, K // group), np.uint16)
    biases = np.zeros((E, rows, K // group), np.uint16)
    for e in (range(E) if experts is None else experts):
        w = gen_weight(cfg, layer, proj, rows, K, index=int(e), bits=bits, group=group)
        codes[e], scales[e], biases[e] = w.codes, w.scales, w.biases
    return U4Weight(codes, scales, biases, bits)


# ---- workload shapes -------------------------------------------------------

@dataclass(frozen=True)
class DecodeShape:
    name: str
    K: int            # hidden size (input width of QKV and gate+up)
    q_out: int
    kv_out: int
    I: int            # intermediate size (gate and up each have I rows)

    @property
    def qkv_rows(self) -> int:
        return self.q_out + 2 * self.kv_out


TINY_QKV = DecodeShape("tiny fused QKV decode (hidden 512, q 512, kv 128)", 512, 512, 128, 0)
DENSE_14B = DecodeShape("14B-shaped decode (hidden 5120, 40 q / 8 kv heads x 128, intermediate 13824)",
                        5120, 5120, 1024, 13824)
DENSE_24B = DecodeShape("24B-dense-shaped decode (hidden 5120, q 4096, kv 1024, intermediate 32768)",
                        5120, 4096, 1024, 32768)
PREFILL_M = 2048
DOUBLED_Q = DecodeShape("doubled-Q QKV (hidden 5120, q 24x256x2, kv 4x256)", 5120, 12288, 1024, 0)


@dataclass(frozen=True)
class RopeShape:
    name: str
    K: int
    n_q: int
    n_kv: int
    head_dim: int
    q_gate: bool
    rot: int
    base: float

    @property
    def rows(self) -> int:
        return (self.n_q * (2 if self.q_gate else 1) + 2 * self.n_kv) * self.head_dim


ROPE_14B = RopeShape("14B-shaped QKV + RoPE (hidden 5120, 40 q / 8 kv heads x 128, full rotary, base 1e6)",
                     5120, 40, 8, 128, False, 128, 1.0e6)
ROPE_GATED = RopeShape("doubled-Q QKV + RoPE (hidden 5120, 24 q heads x 256 with output gate, 4 kv heads, "
                       "rotary 64 of 256, base 1e7)", 5120, 24, 4, 256, True, 64, 1.0e7)
ROPE_MAX_POS = 32768


@dataclass(frozen=True)
class MoEShape:
    name: str
    hidden: int
    E: int
    I: int
    topk: int


MOE_35B = MoEShape("35B-A3B-shaped MoE decode (hidden 2048, 256 experts, I 512, top-8)", 2048, 256, 512, 8)
MOE_PREFILL_M = 2048   # tokens of the routed-expert prefill workload

# config ids used as the first seed word
CFG_TINY, CFG_14B, CFG_24B, CFG_PREFILL, CFG_MOE, CFG_TEST = 1, 2, 3, 4, 5, 9
