"""CPU oracle for the group-wise affine u4 quantized matmul (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library; its only common ground with it is the
seeded input generator in `synth/`.

What is computed, and where the pages state it:
  * Weights are 4-bit integer codes in groups of 64 along the input axis, each
    group with one bf16 scale and one bf16 bias ("Sanctum-MLX", server section:
    4-bit QuantizedLinear with group size 64; saragossa README, quantization
    formats: MLX affine integer weights, bf16 scales/biases, u4 at ~4.5 bits per
    weight).  The dequantized weight is w = scale * q + bias with q in 0..15.
  * Eight codes share one uint32 along the input axis: the fused QKV weight is
    [q_out + 2*kv_out, hidden/8] ("The Cathedral Doubled Itself", the two
    fusions).  Inside a word, input k = 8*w + j sits at bits 4j..4j+3
    (least-significant nibble first).  The pages do not state the nibble order;
    this is the reading taken, and its agreement with MLX's own order is
    parity unpinned (no MLX code or vectors are available).
  * Fused QKV = one matmul over the row-concatenated q/k/v weights, split into
    Q, K, V; fused gate+up = one matmul over [gate; up] followed by
    silu(gate) * up ("The Cathedral Doubled Itself", the two fusions).  Because
    fusion only concatenates rows, the fused result is exactly the plain
    definition y = x . W^T evaluated per row, which is what this module does.
  * The routed-expert variant gathers each selected expert's rows in place from
    a 3-D expert grid ("Sanctum-MLX", server section, switch_mlp; "Four Candles
    for the Cathedral", what's not in this batch).

Dequantization to fp64 is exact: s*q has at most 12 significant bits and the
bias adds a few more, far below 53.  The dot product uses NumPy's fp64 matmul
(a library primitive) on row blocks to bound memory.

Tolerance (the acceptance rule for a GPU value g against oracle value y):
    |g - y| <= 1e-3 * A,   A = sum_k |x_k| * |w_k|  (+ |lin_bias| if present),
evaluated on the GPU's fp32 output before any bf16 rounding: the stated rule, with
nothing added, for every workload.  Two documented additions exist for cases where
the stated rule asks for more than any fp32 evaluation of the design can deliver:
  * `eval_floor`: rows whose weights are all exactly zero while their codes are not
    (constant codes 8 with bias -8*scale) make A = 0, so the rule would demand an exact
    zero; the per-group scale/bias reuse evaluates s*sum(x q) + b*sum(x) in fp32, which
    cannot promise one.  The floor is the worst-case first-order error bound of that
    evaluation, derived in `eval_floor`; only tests of such degenerate rows add it.
  * `bf16_weights=True`: a kernel that rounds each dequantized weight to bf16 before
    multiplying (the prefill design) adds the exact bound of that rounding,
    sum |x| |w - bf16(w)|; at short K (K < 512) the stated rule alone can sit below
    that one rounding for a few elements per million, so only short-K tests add it.
Derived outputs (SwiGLU, expert combine) carry the propagated bounds computed below.
"""
from __future__ import annotations

import numpy as np

GROUP = 64
REL_TOL = 1e-3
FP32_U = 2.0 ** -24          # unit roundoff of fp32 (round to nearest)
# max |d/dg silu(g)| = max sigma(g) * (1 + g * (1 - sigma(g))) ~= 1.09985 (at g ~= 2.40)
SILU_LIPSCHITZ = 1.0999
# relative allowance for the GPU's own fp32 evaluation of silu(g) * u
SWIGLU_EVAL_REL = 2.0 ** -20


# ---- formats ---------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64.  A bf16 value is the top half of the
    fp32 with the same bits, so widen to 32 bits, shift up 16 and read as fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # signalling NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def unpack_u4(codes) -> np.ndarray:
    """uint32 words [..., K/8] -> codes [..., K] (int64), least-significant nibble first."""
    c = np.asarray(codes, dtype=np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    q = (c[..., None] >> shifts) & np.uint32(0xF)
    return q.reshape(*c.shape[:-1], c.shape[-1] * 8).astype(np.int64)


def unpack_bits(codes, bits: int) -> np.ndarray:
    """uint32 words [..., K*bits/32] -> codes [..., K] (int64) for any code width: the row is
    one bit stream (bit j of the stream = bit j % 32 of word j // 32) and code k is stream
    bits [bits*k, bits*k + bits), least-significant bit first, so 3- and 6-bit codes may
    straddle two words.  The saragossa README lists affine integer weights u2/u3/u4/u6/u8
    ("Quantization formats"); the pages do not state the packing, and this plain bit
    stream, which is the 4-bit order of `unpack_u4` at bits = 4, is the reading taken."""
    c = np.ascontiguousarray(np.asarray(codes, dtype="<u4"))
    stream = np.unpackbits(c.view(np.uint8), axis=-1, bitorder="little")
    K = stream.shape[-1] // bits
    f = stream[..., :K * bits].reshape(*stream.shape[:-1], K, bits).astype(np.int64)
    return (f << np.arange(bits, dtype=np.int64)).sum(axis=-1)


E4M3 = "e4m3"


def e4m3_to_f64(q) -> np.ndarray:
    """fp8 e4m3 codes (0..255) -> fp64 from the format's definition: sign bit 7, exponent
    bits 3..6 with bias 7, 3 fraction bits; exponent 0 is subnormal (m/8 * 2^-6); the
    all-ones pattern S.1111.111 is NaN (no infinities)."""
    q = np.asarray(q, dtype=np.int64)
    sign = np.where(q & 0x80, -1.0, 1.0)
    e = (q >> 3) & 0xF
    m = (q & 0x7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    v = np.where((e == 15) & (q & 0x7 == 7), np.nan, v)
    return sign * v


def code_values(codes, bits) -> np.ndarray:
    """The value each code stands for: the integer q for bits 2..8, the e4m3 number for
    bits = E4M3 (8-bit codes; the saragossa README lists fp8 e4m3 next to the integer
    widths, "Quantization formats", without its scaling; the reading taken is the same
    affine form with the e4m3 value in place of q)."""
    if bits == E4M3:
        return e4m3_to_f64(unpack_bits(codes, 8))
    return (unpack_u4(codes) if bits == 4 else unpack_bits(codes, bits)).astype(np.float64)


def storage_bits(bits) -> int:
    return 8 if bits == E4M3 else int(bits)


def dequant(codes, scales, biases, bits=4) -> np.ndarray:
    """W[n, k] = s[n, k // G] * q[n, k] + b[n, k // G] in fp64, shape [rows, K], with the
    group size G = K / (scales per row) (64 on the workloads; 32 to 128 on the pages:
    saragossa README, "Capabilities"); q is the code's value (`code_values`)."""
    q = code_values(codes, bits)
    K = q.shape[-1]
    s = bf16_to_f64(scales)
    b = bf16_to_f64(biases)
    G = K // s.shape[-1]
    if s.shape[-1] * G != K or b.shape != s.shape:
        raise ValueError("scales/biases must be [rows, K/G]")
    s_k = np.repeat(s, G, axis=-1)
    b_k = np.repeat(b, G, axis=-1)
    return s_k * q + b_k


# ---- plain projection --------------------------------------------------------

def project(x_bits, codes, scales, biases, lin_bias=None, row_block: int = 1024, bf16_weights: bool = False,
            bits: int = 4):
    """y[m, n] = sum_k x[m, k] * W[n, k] (+ lin_bias[n]) in fp64, with the magnitude sums
    the tolerance is built from:
      A[m, n] = sum_k |x[m, k]| * |W[n, k]|  (+ |lin_bias[n]|)
      S[m, n] = sum_k |x[m, k]| * |s[n, k // G]|    (activation mass weighted by the scale,
                                                     i.e. the size of a one-code change)
      B[m, n] = sum_k |x[m, k]| * |b[n, k // G]|    (the same for the bias)
    and, with bf16_weights, R[m, n] = sum_k |x[m, k]| * |W[n, k] - bf16(W[n, k])| (the
    largest effect of rounding every dequantized weight to bf16, RNE) as a fifth value.
    x_bits: bf16 bits [M, K] (or [K]); codes [N, K*bits/32]; scales/biases [N, K/G];
    lin_bias: optional bf16 bits [N]."""
    x = bf16_to_f64(x_bits)
    squeeze = x.ndim == 1
    if squeeze:
        x = x[None, :]
    N = codes.shape[0]
    K = x.shape[1]
    if codes.shape[1] * 32 != K * storage_bits(bits):
        raise ValueError("x width must equal 32/bits * words per row")
    G = K // scales.shape[1]
    y = np.empty((x.shape[0], N))
    A = np.empty((x.shape[0], N))
    R = np.zeros((x.shape[0], N))
    ax = np.abs(x)
    xg = ax.reshape(x.shape[0], K // G, G).sum(axis=2)                  # [M, K/G]
    S = xg @ np.abs(bf16_to_f64(scales)).T
    B = xg @ np.abs(bf16_to_f64(biases)).T
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        W = dequant(codes[r0:r1], scales[r0:r1], biases[r0:r1], bits)
        y[:, r0:r1] = x @ W.T
        A[:, r0:r1] = ax @ np.abs(W).T
        if bf16_weights:
            R[:, r0:r1] = ax @ np.abs(W - bf16_to_f64(f32_to_bf16_bits(W))).T
    if lin_bias is not None:
        lb = bf16_to_f64(lin_bias)
        y += lb[None, :]
        A += np.abs(lb)[None, :]
    out = (y, A, S, B, R) if bf16_weights else (y, A, S, B)
    if squeeze:
        return tuple(v[0] for v in out)
    return out


def tolerance(A) -> np.ndarray:
    """Acceptance bound of one projection output: the stated rule, 1e-3 * sum|x w|."""
    return REL_TOL * np.asarray(A)


def eval_floor(S, B) -> np.ndarray:
    """Worst-case first-order error of evaluating one 4-bit projection output in fp32 the
    way the decode design does (per-group scale/bias reuse, "Sanctum-MLX" and the pages'
    affine u4 format; the bias term reduces to b * sum(x)), for rows where the stated rule
    demands an exact zero.  S = sum_k |x_k| |s_k|, B = sum_k |x_k| |b_k|.

    Per chunk of 32 inputs with scale s and bias b the value is t = s*(D - 128 X) + b*X,
    D = sum x (128 + q) and X = sum x, each a chain of 32 products (exact in fp32: bf16
    times an 8-bit integer) added with at most 32 roundings; a rounding of a partial sum
    of terms bounded by T costs at most u*T, u = 2^-24.  So
        |D - D*| <= 32 u (128 + 15) sum|x|,     |X - X*| <= 32 u sum|x|,
        |fl(D - 128 X) - sum x q| <= (32*143 + 128*32 + 15) u sum|x| = 8687 u sum|x|,
    and t adds |b| 32 u sum|x|.  Accumulating the chunk terms of a row (two fused
    multiply-adds per chunk, at most 5 chunks per lane, 5 lane-sum steps, up to 16 K
    slices: at most 31 roundings of partial sums bounded by sum (15|s| + |b|) |x|) adds
    31 u (15 S + B).  Total: (8687 + 465) u S + (32 + 31) u B = 9152 u S + 63 u B."""
    return FP32_U * (9152.0 * np.asarray(S) + 63.0 * np.asarray(B))


def linear(x_bits, codes, scales, biases, lin_bias=None, row_block: int = 1024, bf16_weights: bool = False,
           bits: int = 4, floor: bool = False):
    """(y, tol) of one projection; tol = 1e-3 * sum|x w| (`tolerance`).  With bf16_weights
    (a kernel that rounds each dequantized weight to bf16 before multiplying, as the
    prefill design does) tol also carries R = sum |x| |w - bf16(w)|, the bound of that
    rounding; with floor (rows of exactly zero weights) the fp32 evaluation floor
    `eval_floor` of the 4-bit decode design."""
    out = project(x_bits, codes, scales, biases, lin_bias, row_block, bf16_weights=bf16_weights, bits=bits)
    y, A, S, B = out[:4]
    t = tolerance(A)
    if floor:
        t = t + eval_floor(S, B)
    if bf16_weights:
        t = t + out[4]
    return y, t


# ---- fused QKV -------------------------------------------------------------

def fused_qkv(x_bits, codes, scales, biases, q_out: int, kv_out: int, lin_bias=None, bf16_weights: bool = False,
              bits: int = 4):
    """Rows [0, q_out) -> Q, [q_out, q_out+kv_out) -> K, [q_out+kv_out, q_out+2kv_out) -> V.
    Returns ((q, k, v), (tq, tk, tv)): values and per-element tolerances."""
    if codes.shape[0] != q_out + 2 * kv_out:
        raise ValueError("fused QKV weight must have q_out + 2*kv_out rows")
    y, t = linear(x_bits, codes, scales, biases, lin_bias, bf16_weights=bf16_weights, bits=bits)
    a, b = q_out, q_out + kv_out
    return (y[..., :a], y[..., a:b], y[..., b:]), (t[..., :a], t[..., a:b], t[..., b:])


# ---- fused QKV with rotary position embedding ------------------------------------
#
# The pages' unshipped second phase does the split of the fused QKV output and its
# rotary position embedding in one kernel ("Sanctum-MLX", shipped phases table, Phase 2;
# "The Cathedral Doubled Itself", the kernel that worked and the kernel that won't).  The
# pages do not spell the rotation out; the readings taken here:
#   * each head of head_dim rows is rotated in the half-split form: for i < rot/2 the
#     pair (a, b) = (d_i, d_{i + rot/2}) becomes (a c - b s, b c + a s), dims [rot,
#     head_dim) pass through (rot = head_dim is full rotary);
#   * c, s come from a table cos_sin[p, i], cos_sin[p, rot/2 + i] (fp32) at the token's
#     position p = positions[m]; the table is an input, built once by the caller;
#   * Q and K heads are rotated, V heads are not;
#   * with q_gate the Q section holds, per query head, head_dim query rows followed by
#     head_dim output-gate rows ("The Cathedral Doubled Itself", the 35B port: the
#     qwen3_5 q projection carries queries and gate together); the gate is not rotated.

ROPE_EVAL_REL = 2.0 ** -21   # the GPU's fp32 evaluation of a c - b s (two products, one sum)


def rope_head_rows(n_q: int, n_kv: int, head_dim: int, q_gate: bool):
    """Row ranges of the fused weight: list of (kind, head, first_row) for every head, kind
    in 'q', 'gate', 'k', 'v', in weight order."""
    out = []
    r = 0
    for h in range(n_q):
        out.append(("q", h, r))
        r += head_dim
        if q_gate:
            out.append(("gate", h, r))
            r += head_dim
    for kind in ("k", "v"):
        for h in range(n_kv):
            out.append((kind, h, r))
            r += head_dim
    return out, r


def rope_rotate(a, b, c, s):
    """Half-split rotation of the pairs (a, b) by the angle whose cosine and sine are c, s."""
    return a * c - b * s, b * c + a * s


def qkv_rope(x_bits, codes, scales, biases, n_q: int, n_kv: int, head_dim: int, q_gate: bool, rot: int,
             positions, cos_sin, lin_bias=None, bf16_weights: bool = False):
    """Fused QKV projection, split into heads, Q and K heads rotated at each token's
    position.  x_bits [M, K]; positions int [M]; cos_sin fp32 [max_pos, rot].
    Returns ((q, gate, k, v), (tq, tg, tk, tv)), each [M, heads, head_dim] (gate None
    unless q_gate); tolerances propagate the projection's through the rotation:
    |c| t_a + |s| t_b, plus the GPU's fp32 evaluation (ROPE_EVAL_REL)."""
    heads, rows = rope_head_rows(n_q, n_kv, head_dim, q_gate)
    if codes.shape[0] != rows or head_dim % 2 or rot % 2 or not 0 < rot <= head_dim:
        raise ValueError("inconsistent rotary QKV shape")
    x = np.atleast_2d(np.asarray(x_bits))
    y, t = linear(x, codes, scales, biases, lin_bias, bf16_weights=bf16_weights)
    M = x.shape[0]
    pos = np.asarray(positions, dtype=np.int64).reshape(M)
    cs = np.asarray(cos_sin, dtype=np.float32).astype(np.float64)
    half = rot // 2
    c = cs[pos, :half][:, None, :]          # [M, 1, half]
    s = cs[pos, half:rot][:, None, :]
    out = {k: np.zeros((M, n_q if k in ("q", "gate") else n_kv, head_dim)) for k in ("q", "gate", "k", "v")}
    tol = {k: np.zeros_like(v) for k, v in out.items()}
    for kind, h, r0 in heads:
        out[kind][:, h, :] = y[:, r0:r0 + head_dim]
        tol[kind][:, h, :] = t[:, r0:r0 + head_dim]
    for kind in ("q", "k"):
        v, tv = out[kind], tol[kind]
        a, b = v[..., :half].copy(), v[..., half:rot].copy()
        ta, tb = tv[..., :half].copy(), tv[..., half:rot].copy()
        ra, rb = rope_rotate(a, b, c, s)
        v[..., :half], v[..., half:rot] = ra, rb
        ev = ROPE_EVAL_REL * (np.abs(a * c) + np.abs(b * s) + np.abs(b * c) + np.abs(a * s))
        tv[..., :half] = np.abs(c) * ta + np.abs(s) * tb + ev
        tv[..., half:rot] = np.abs(c) * tb + np.abs(s) * ta + ev
    g = out["gate"] if q_gate else None
    tg = tol["gate"] if q_gate else None
    return (out["q"], g, out["k"], out["v"]), (tol["q"], tg, tol["k"], tol["v"])


# ---- SwiGLU ------------------------------------------------------------------

def sigmoid(g) -> np.ndarray:
    """Logistic function, evaluated without overflow: e^{min(g,0)} / (1 + e^{-|g|})."""
    g = np.asarray(g, dtype=np.float64)
    return np.exp(np.minimum(g, 0.0)) / (1.0 + np.exp(-np.abs(g)))


def silu(g) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g)


def swiglu(g, u) -> np.ndarray:
    """h = silu(gate) * up (the activation applied after the two parallel matmuls)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def swiglu_tol(g, u, tg, tu) -> np.ndarray:
    """Bound on |h_gpu - h| when the GPU's gate and up are within tg, tu of g, u:
    |silu(g')u' - silu(g)u| <= L*tg*(|u|+tu) + |silu(g)|*tu, plus the GPU's fp32
    evaluation of silu and the product (SWIGLU_EVAL_REL relative)."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    h = swiglu(g, u)
    return (SILU_LIPSCHITZ * tg * (np.abs(u) + tu) + np.abs(silu(g)) * tu
            + SWIGLU_EVAL_REL * (np.abs(h) + SILU_LIPSCHITZ * tg * (np.abs(u) + tu) + np.abs(silu(g)) * tu))


def gate_up_swiglu(x_bits, codes, scales, biases, I: int, bf16_weights: bool = False, bits: int = 4):
    """Rows [0, I) are gate, [I, 2I) are up.  Returns (h, tol_h)."""
    if codes.shape[0] != 2 * I:
        raise ValueError("fused gate+up weight must have 2*I rows")
    y, t = linear(x_bits, codes, scales, biases, bf16_weights=bf16_weights, bits=bits)
    g, u = y[..., :I], y[..., I:]
    tg, tu = t[..., :I], t[..., I:]
    return swiglu(g, u), swiglu_tol(g, u, tg, tu)


# ---- routed experts ------------------------------------------------------------

def moe_gate_up(x_bits, grid_codes, grid_scales, grid_biases, expert_ids, rows: int, bits: int = 4):
    """Stage 1: for slot k, expert e = ids[k] in [0, E): h[k] = silu(G_e x) * (U_e x) over
    rows [0, rows/2) (gate) and [rows/2, rows) (up) of grid[e].  An id outside [0, E)
    means no expert: h[k] = 0.  Returns (h [topk, rows/2], tol)."""
    E = grid_codes.shape[0]
    I = rows // 2
    topk = len(expert_ids)
    h = np.zeros((topk, I))
    t = np.zeros((topk, I))
    for k, e in enumerate(np.asarray(expert_ids).tolist()):
        if 0 <= e < E:
            hk, tk = gate_up_swiglu(np.asarray(x_bits).reshape(-1), grid_codes[e], grid_scales[e],
                                    grid_biases[e], I, bits=bits)
            h[k], t[k] = hk, tk
    return h, t


def moe_down_combine(h_bits, grid_codes, grid_scales, grid_biases, expert_ids, expert_w, bits: int = 4):
    """Stage 2: y = sum_k p_k * (D_{ids[k]} h_k), k in increasing order; ids outside [0, E)
    contribute nothing.  h_bits: bf16 bits [topk, K] of the stage-1 output fed to both
    sides; p: the fp32 combine weights.  Returns (y, tol)."""
    E = grid_codes.shape[0]
    rows = grid_codes.shape[1]
    y = np.zeros(rows)
    t = np.zeros(rows)
    p = np.asarray(expert_w, dtype=np.float32).astype(np.float64)
    for k, e in enumerate(np.asarray(expert_ids).tolist()):
        if 0 <= e < E:
            yk, tk = linear(np.asarray(h_bits)[k], grid_codes[e], grid_scales[e], grid_biases[e], bits=bits)
            y += p[k] * yk
            t += abs(p[k]) * tk
    return y, t


def moe_prefill_gate_up(x_bits, grid_codes, grid_scales, grid_biases, expert_ids, rows: int,
                        bf16_weights: bool = False):
    """Stage 1 over a batch of tokens (prefill): for token m and slot k with expert
    e = ids[m, k] in [0, E), h[m, k] = silu(G_e x_m) * (U_e x_m); other pairs get h = 0.
    Computed expert by expert, as the pages' in-place expert grid is meant to be used:
    the (token, slot) pairs routed to e are gathered and their tokens multiplied by the
    gate+up rows of grid[e] in one product.  bf16_weights adds the exact effect of feeding
    bf16-rounded weights (a kernel that multiplies on the matrix cores).
    Returns (h [M, topk, rows/2], tol)."""
    x = np.asarray(x_bits)
    ids = np.asarray(expert_ids)
    M, topk = ids.shape
    E = grid_codes.shape[0]
    I = rows // 2
    h = np.zeros((M, topk, I))
    t = np.zeros((M, topk, I))
    for e in range(E):
        m_idx, k_idx = np.nonzero(ids == e)
        if len(m_idx) == 0:
            continue
        he, te = gate_up_swiglu(x[m_idx], grid_codes[e], grid_scales[e], grid_biases[e], I,
                                bf16_weights=bf16_weights)
        h[m_idx, k_idx] = he
        t[m_idx, k_idx] = te
    return h, t


def moe_prefill_down_combine(h_bits, grid_codes, grid_scales, grid_biases, expert_ids, expert_w,
                             bf16_weights: bool = False):
    """Stage 2 over a batch of tokens: y[m] = sum_k p[m, k] * (D_e h[m, k]) with
    e = ids[m, k]; pairs with no expert contribute nothing.  h_bits: bf16 bits
    [M, topk, K] fed to both sides; p: the fp32 combine weights [M, topk].  Computed
    expert by expert (gathered h rows times grid[e]), then added per token.  Returns
    (y [M, rows], tol) with tol = sum_k |p| * tol(D_e h[m, k])."""
    hb = np.asarray(h_bits)
    ids = np.asarray(expert_ids)
    M, topk = ids.shape
    E, rows = grid_codes.shape[0], grid_codes.shape[1]
    p = np.asarray(expert_w, dtype=np.float32).astype(np.float64)
    y = np.zeros((M, rows))
    t = np.zeros((M, rows))
    for e in range(E):
        m_idx, k_idx = np.nonzero(ids == e)
        if len(m_idx) == 0:
            continue
        ye, te = linear(hb[m_idx, k_idx], grid_codes[e], grid_scales[e], grid_biases[e],
                        bf16_weights=bf16_weights)
        pe = p[m_idx, k_idx][:, None]
        np.add.at(y, m_idx, pe * ye)
        np.add.at(t, m_idx, np.abs(pe) * te)
    return y, t


def f32_to_bf16_bits(v) -> np.ndarray:
    """Round fp64/fp32 values to fp32 and then to bf16 (round to nearest, ties to even)
    by integer arithmetic on the fp32 bit pattern; NaN is not expected here."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)
