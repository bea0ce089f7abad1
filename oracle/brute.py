"""Brute-force definition of the quantized projection, pure Python (no NumPy).

TEST INFRASTRUCTURE ONLY (pins the NumPy oracle; never imported by the
product path).  It works from the *unpacked* definition of the format: it is
handed the integer codes and the bf16 scale/bias bit patterns, decodes each
bf16 from the IEEE-style field definition (sign, 8-bit biased exponent, 7-bit
fraction), forms w = s*q + b per input and sums x*w with math.fsum (exactly
rounded), so a reader can check every step by eye.  The definitions follow
"Sanctum-MLX" (server section: 4-bit, group size 64) and the saragossa README
(quantization formats: affine integer weights with bf16 scales/biases).
"""
from __future__ import annotations

import math


def bf16_value(bits: int) -> float:
    """Decode a bf16 bit pattern from its fields: (-1)^s * 2^(e-127) * (1 + f/128),
    subnormals 2^-126 * f/128, e == 255 -> inf/nan."""
    bits &= 0xFFFF
    s = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0:
        return s * math.ldexp(f / 128.0, -126)
    if e == 255:
        return s * math.inf if f == 0 else math.nan
    return s * math.ldexp(1.0 + f / 128.0, e - 127)


def bf16_bits(sign: int, exp: int, frac: int) -> int:
    """Assemble a bf16 bit pattern from its fields."""
    return ((sign & 1) << 15) | ((exp & 0xFF) << 7) | (frac & 0x7F)


def pack_row(codes_row) -> list:
    """Pack a row of 4-bit codes (length K, K % 8 == 0) into uint32 words with
    code k in word k // 8 at weight 16**(k % 8) (least-significant nibble first)."""
    words = []
    for w in range(len(codes_row) // 8):
        v = 0
        for j in range(8):
            q = int(codes_row[8 * w + j])
            assert 0 <= q <= 15
            v += q * (16 ** j)
        words.append(v)
    return words


def pack_row_bits(codes_row, bits: int) -> list:
    """Pack a row of `bits`-bit codes into uint32 words as one little-endian bit stream:
    the row is the integer sum of q_k * 2**(bits*k), and word w holds its bits
    [32w, 32w + 32).  Any width; a code may straddle two words."""
    v = 0
    for k, q in enumerate(codes_row):
        q = int(q)
        assert 0 <= q < 2 ** bits
        v += q << (bits * k)
    n = len(codes_row) * bits // 32
    assert n * 32 == len(codes_row) * bits
    return [(v >> (32 * w)) & 0xFFFFFFFF for w in range(n)]


def project(x_bits, q, s_bits, b_bits, group: int = 64, lin_bias_bits=None):
    """y[m][n] = sum_k x[m][k] * (s[n][k//group] * q[n][k] + b[n][k//group]) (+ lin_bias[n]).

    x_bits: list of M lists of K bf16 patterns; q: list of N lists of K ints;
    s_bits, b_bits: N lists of K/group bf16 patterns.  Returns (y, A) as lists of lists,
    A = sum_k |x||w| (+ |lin_bias|)."""
    M, N = len(x_bits), len(q)
    y = [[0.0] * N for _ in range(M)]
    A = [[0.0] * N for _ in range(M)]
    for m in range(M):
        xv = [bf16_value(v) for v in x_bits[m]]
        for n in range(N):
            terms = []
            for k in range(len(xv)):
                g = k // group
                w = bf16_value(s_bits[n][g]) * q[n][k] + bf16_value(b_bits[n][g])
                terms.append(xv[k] * w)
            if lin_bias_bits is not None:
                terms.append(bf16_value(lin_bias_bits[n]))
            y[m][n] = math.fsum(terms)
            A[m][n] = math.fsum(abs(t) for t in terms)
    return y, A


def silu(g: float) -> float:
    """g * logistic(g), written from the definition with the overflow-free branch."""
    if g >= 0:
        return g / (1.0 + math.exp(-g))
    e = math.exp(g)
    return g * e / (1.0 + e)
