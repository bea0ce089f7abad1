// Device helpers shared by the u4 group-64 affine kernels (gfx950 / CDNA4).
//
// Weight format (the library's input contract): eight 4-bit codes per uint32
// along the input axis, code k of a row at bits 4*(k%8)..+3 of word k/8, and one
// bf16 scale and one bf16 bias per 64 inputs, w = scale*q + bias.  The 4-bit,
// group-64, bf16 scale/bias format is stated in "Sanctum-MLX" (server section)
// and the saragossa README (quantization formats); the hidden/8 packing in
// "The Cathedral Doubled Itself" (the two fusions).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagicPair = 0x43004300u;  // bf16 pair (128.0, 128.0)

// Raw buffer descriptors: loads at offsets >= num_records return zero, which is how
// the kernels treat the ragged end of a row, a K slice or a buffer.  The range check
// is per dword, so every buffer read here is dword-aligned and dword-sized or a bf16.
constexpr int kBufferFlags = 0x00020000;  // dword 3 of a gfx9 raw buffer descriptor (32-bit data)
constexpr int kLoadNT = 2;                // aux bit: non-temporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : uint32_t(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(n), kBufferFlags);
}
constexpr uint32_t kNibblePair = 0x000F000Fu;

// Keep a constant in a VGPR so that v_and_or_b32 can take it alongside an SGPR mask
// (a gfx9 VOP3 instruction reads at most one scalar operand and no literal).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> one dword of two bf16 (RNE), low half first (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Nibble pair t (t = 0..3) of a code word as the exact bf16 pair (128+q_t, 128+q_{t+4}):
// the bf16 pattern 0x43 0x0q is 128 + q, since the ulp at 128 is 1.
__device__ __forceinline__ uint32_t nib_pair(uint32_t w, int t, uint32_t magic) {
  return ((w >> (4 * t)) & kNibblePair) | magic;
}

// Activations of one 32-code chunk, permuted to match nib_pair: xp[4*j + t] holds
// (x[8j+t], x[8j+t+4]) for word j = 0..3, t = 0..3.  d[m] holds (x[2m], x[2m+1]).
__device__ __forceinline__ void permute_chunk(const uint32_t d[16], uint32_t xp[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    xp[4 * j + 0] = __builtin_amdgcn_perm(d[4 * j + 2], d[4 * j + 0], 0x05040100u);
    xp[4 * j + 1] = __builtin_amdgcn_perm(d[4 * j + 2], d[4 * j + 0], 0x07060302u);
    xp[4 * j + 2] = __builtin_amdgcn_perm(d[4 * j + 3], d[4 * j + 1], 0x05040100u);
    xp[4 * j + 3] = __builtin_amdgcn_perm(d[4 * j + 3], d[4 * j + 1], 0x07060302u);
  }
}

// Sum of the 32 activations of a chunk, by the same chain of dot2 operations (against
// (1,1)) that chunk_dot128 uses against (128+q).  With all codes zero the two chains
// differ by an exact factor 128, so q == 0 yields exactly zero after subtraction.
__device__ __forceinline__ float chunk_xsum(const uint32_t xp[16]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s = dot2_bf16(xp[i], 0x3F803F80u, s);
  return s;
}

// sum_k x_k * (128 + q_k) over one chunk (four code words), fp32.
__device__ __forceinline__ float chunk_dot128(const uint32_t (&w)[4], const uint32_t xp[16], uint32_t magic) {
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int t = 0; t < 4; ++t) d = dot2_bf16(nib_pair(w[j], t, magic), xp[4 * j + t], d);
  }
  return d;
}

// ---- code widths of the affine family ------------------------------------------------
// A row is one little-endian bit stream of `BITS`-bit codes, so a chunk of 32 codes is
// BITS words.  Codec<BITS> turns a chunk's words into exact bf16 pairs (128 + q_a,
// 128 + q_b) for v_dot2 against activation pairs permuted to the same order, and
// returns sum_k x_k q_k of the chunk (fp32).  `d[m]` below holds (x[2m], x[2m+1]).
//
// Activation pair (x[a], x[b]) from the unpermuted pairs.
__device__ __forceinline__ uint32_t x_pair(const uint32_t d[16], int a, int b) {
  const uint32_t sel = ((b & 1) ? 0x07060000u : 0x05040000u) | ((a & 1) ? 0x0302u : 0x0100u);
  return __builtin_amdgcn_perm(d[b >> 1], d[a >> 1], sel);
}
// Bits [s, s + 32) of the stream of words w[] (s a compile-time constant after unrolling;
// words past the chunk read as `pad`).
template <int NW>
__device__ __forceinline__ uint32_t stream_window(const uint32_t (&w)[NW], int s) {
  const int i = s >> 5, sh = s & 31;
  const uint32_t lo = i < NW ? w[i] : 0u;
  if (sh == 0) return lo;
  const uint32_t hi = i + 1 < NW ? w[i + 1] : 0u;
  return __builtin_amdgcn_alignbit(hi, lo, sh);
}

template <int BITS>
struct Codec;

// 4 bits: pair (q_{8j+t}, q_{8j+t+4}) of word j is one shift-and-or (nib_pair).
template <>
struct Codec<4> {
  static constexpr int kWords = 4;
  static __device__ __forceinline__ void permute(const uint32_t d[16], uint32_t xp[16]) { permute_chunk(d, xp); }
  static __device__ __forceinline__ float dot_q(const uint32_t (&w)[4], const uint32_t xp[16], float xs,
                                                uint32_t magic) {
    return fmaf(-128.0f, xs, chunk_dot128(w, xp, magic));
  }
};

// 8 bits: each byte q = 16 h + l is taken as its two nibbles; pairs (l_{4j+u}, l_{4j+u+2})
// and (h_{4j+u}, h_{4j+u+2}) of word j share the activation pair (x_{4j+u}, x_{4j+u+2}).
template <>
struct Codec<8> {
  static constexpr int kWords = 8;
  static __device__ __forceinline__ void permute(const uint32_t d[16], uint32_t xp[16]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xp[2 * j] = x_pair(d, 4 * j, 4 * j + 2);
      xp[2 * j + 1] = x_pair(d, 4 * j + 1, 4 * j + 3);
    }
  }
  static __device__ __forceinline__ float dot_q(const uint32_t (&w)[8], const uint32_t xp[16], float xs,
                                                uint32_t magic) {
    float dl = 0.f, dh = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dl = dot2_bf16((w[j] & kNibblePair) | magic, xp[2 * j], dl);
      dl = dot2_bf16(((w[j] >> 8) & kNibblePair) | magic, xp[2 * j + 1], dl);
      dh = dot2_bf16(((w[j] >> 4) & kNibblePair) | magic, xp[2 * j], dh);
      dh = dot2_bf16(((w[j] >> 12) & kNibblePair) | magic, xp[2 * j + 1], dh);
    }
    // sum x q = 16 (dh - 128 xs) + (dl - 128 xs); each difference is exactly 0 for zero codes
    return fmaf(16.0f, fmaf(-128.0f, xs, dh), fmaf(-128.0f, xs, dl));
  }
};

// 2 bits: pair (q_{16j+t}, q_{16j+t+8}) of word j: ((w >> 2t) & 0x00030003) | magic.
template <>
struct Codec<2> {
  static constexpr int kWords = 2;
  static __device__ __forceinline__ void permute(const uint32_t d[16], uint32_t xp[16]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 8; ++t) xp[8 * j + t] = x_pair(d, 16 * j + t, 16 * j + t + 8);
  }
  static __device__ __forceinline__ float dot_q(const uint32_t (&w)[2], const uint32_t xp[16], float xs,
                                                uint32_t magic) {
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 8; ++t) d = dot2_bf16(((w[j] >> (2 * t)) & 0x00030003u) | magic, xp[8 * j + t], d);
    return fmaf(-128.0f, xs, d);
  }
};

// 3 and 6 bits (codes may straddle words): pair (q_k, q_{k+16}); q_k is the low BITS of
// the stream window at BITS*k, q_{k+16} sits at bit 16 of the window at BITS*k + 16*BITS - 16.
template <int BITS>
struct CodecStream {
  static constexpr int kWords = BITS;
  static __device__ __forceinline__ void permute(const uint32_t d[16], uint32_t xp[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) xp[k] = x_pair(d, k, k + 16);
  }
  static __device__ __forceinline__ float dot_q(const uint32_t (&w)[BITS], const uint32_t xp[16], float xs,
                                                uint32_t magic) {
    constexpr uint32_t m = (1u << BITS) - 1u;
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t lo = stream_window(w, BITS * k) & m;
      const uint32_t hi = stream_window(w, BITS * k + 16 * BITS - 16) & (m << 16);
      d = dot2_bf16(lo | hi | magic, xp[k], d);
    }
    return fmaf(-128.0f, xs, d);
  }
};
template <>
struct Codec<3> : CodecStream<3> {};

// fp8 e4m3 codes (8 bits each, word j = codes 4j .. 4j+3): two codes at a time become an
// exact bf16 pair (v_cvt_scalef32_pk_bf16_fp8 with scale 1; bf16 holds every e4m3 value),
// against the activation pairs in their natural order.
struct CodecE4M3 {
  static constexpr int kWords = 8;
  static __device__ __forceinline__ void permute(const uint32_t d[16], uint32_t xp[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) xp[i] = d[i];
  }
  static __device__ __forceinline__ float dot_q(const uint32_t (&w)[8], const uint32_t xp[16], float,
                                                uint32_t) {
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, false),
                                          __builtin_bit_cast(bf16x2_t, xp[2 * j]), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, true),
                                          __builtin_bit_cast(bf16x2_t, xp[2 * j + 1]), d, false);
    }
    return d;
  }
};
template <>
struct Codec<6> : CodecStream<6> {};

// Sum over the LPR lanes of each row slot (LPR = 16 or 32) with DPP.  After return the
// slot's total is in every lane of its last 16-lane row (lanes 16*r + 15 - ... of row r).
template <int LPR>
__device__ __forceinline__ float slot_reduce(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  if constexpr (LPR == 32) {
    // row_bcast:15 into rows 1 and 3: row 1 = row0 + row1, row 3 = row2 + row3
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  }
  return v;
}

// Lane (within the wave) that holds slot s's total after slot_reduce.
template <int LPR>
__device__ __forceinline__ constexpr int slot_result_lane(int s) {
  return LPR == 32 ? 32 * s + 16 : 16 * s;
}

// silu(g) * u, silu(g) = g / (1 + e^-g), with the hardware base-2 exponential and
// reciprocal (each within about an ulp) rather than the full-range expf and the IEEE
// division (~30 more VALU ops per output).  The exponent -g log2(e) is carried as a rounded
// head and its residual (the product's rounding error and the constant's second word),
// applied to first order, so the relative error stays within a few ulp for every g (2.4e-7
// measured over g in [-120, 120] wherever the result is a normal fp32, against 1.8e-7 for
// the expf / division form).  The exponent is capped at 126: beyond it the residual grows
// and e overflows to inf, whose reciprocal 0 gives -0 (as g / (1 + inf) does); below -126
// e is 0 (or denormal) and the result g.
__device__ __forceinline__ float silu_times(float g, float u) {
  constexpr float kLog2e = 1.44269502f;        // log2(e) rounded to fp32
  constexpr float kLog2eLo = 1.925963033e-8f;  // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147181f;
  const float x = fminf(-g * kLog2e, 126.0f);
  const float xl = fmaf(-g, kLog2e, -x) + (-g) * kLog2eLo;
  const float e0 = __builtin_amdgcn_exp2f(x);
  const float e = x > -126.0f ? fmaf(e0, xl * kLn2, e0) : e0;
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, bool f32) {
  if (f32) {
    static_cast<float*>(out)[idx] = v;
  } else {
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  }
}

}  // namespace qmm
