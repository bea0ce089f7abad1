// Small-batch kernel (up to 32 activation rows, and up to 256 where the prefill GEMM's
// grid would be small; M = 2 only where the two-row GEMV does not apply) for the u4
// group-64 affine projections on gfx950.
//
// Between decode (one activation row: weight-bandwidth bound, the GEMV) and prefill
// (hundreds of rows: matrix bound, the LDS-dequant GEMM) the work is still one pass over
// the weights, but every weight now meets up to 16 activation rows per pass.  The GEMV's
// dot2 chain would need every lane to hold 16 activation rows; here the matrix cores
// take the activations instead ("Sanctum-MLX", latency testing: prefill is the matmul
// regime) while the weights stream at the GEMV's rate.
//
// What is computed: y[m][n] = sum_k x[m][k] * (s[n, k/64] * q[n, k] + b[n, k/64]), with the
// fused-QKV split and the SwiGLU epilogue of "The Cathedral Doubled Itself" (the two
// fusions) and the rotary QKV epilogue (qmm_rope.h), for 16 or 32 activation rows per
// block (grid.y covers more).
//
// Layout of the work:
//   * a unit is 16 weight rows (QKV / linear: 16 consecutive rows; SwiGLU: 8 gate rows
//     and their 8 up rows; rotary QKV: the two rows of 8 rotating pairs); a block of S
//     waves walks units with a grid stride, wave s
//     owning the K slice [s*K/S, (s+1)*K/S) of every unit;
//   * the unit's packed codes and its scales and biases go global -> LDS directly
//     (buffer_load ... lds, 1 KB contiguous per wave instruction) into a ring of 2 to 4
//     unit buffers: while unit i is multiplied, the next ones are in flight;
//   * the activations of a wave's slice stay in registers for the whole kernel as
//     v_mfma_f32_16x16x32_bf16 operands (16 rows x 32 inputs per instruction), permuted to
//     the nibble-pair order of the codes;
//   * per 64-input group a lane turns 16 codes of its column into exact bf16 (128 + q)
//     pairs (no rounding of any weight), two MFMAs give D[m][n] = sum x (128 + q) over the
//     group, and the group's scale and bias enter in fp32 as
//     y += s * (D - 128 * xs) + b * xs, with xs[m] = sum x over the group (an MFMA against
//     ones, once per kernel where the registers allow, else once per unit);
//   * the slice partials of a unit meet in LDS and are added in slice order, each output
//     by one lane of one of the waves, after the next unit's barrier (two partial buffers:
//     one barrier per unit) where LDS holds three unit buffers, else after a second one.
// Every output depends only on its own activation row, K and the unit layout, so a row's
// result does not depend on the other rows of the batch or on M.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_rope.h"

namespace qmm {
namespace bmv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kUnit = 16;   // weight rows per unit (the MFMA's columns)
constexpr int kRows = 16;   // activation rows per MFMA tile (a block holds MB tiles)

// LDS of one unit buffer for S waves (K slices) of GPS groups each, K = 64 * S * GPS:
//   codes [16 rows][K/32 chunks of 16 B]; chunk c of row r sits in slot c ^ (r & 15), so
//   the 16 rows a wave reads at one chunk hit 16 different bank groups;
//   scales [16][K/64] bf16, then biases [16][K/64] bf16, each padded to whole KB.
#ifndef QMM_BMV_DEFER
#define QMM_BMV_DEFER 1
#endif
template <int S, int GPS, int MB>
struct Layout {
  static constexpr int kSlices = S;
  static constexpr int K = 64 * S * GPS;
  static constexpr int row_bytes = K / 2;
  static constexpr int code_bytes = kUnit * row_bytes;  // 4 KB * GPS
  static constexpr int sb_row = K / 32;                 // bytes of bf16 scales per row
  static constexpr int sb_bytes = kUnit * sb_row;
  static constexpr int sb_pad = (sb_bytes + 1023) / 1024 * 1024;
  static constexpr int buf_bytes = code_bytes + 2 * sb_pad;
  static constexpr int code_dma = code_bytes / 1024;  // 1 KB wave instructions per unit
  static constexpr int sb_dma = sb_pad / 1024;
  // wave s requests code instructions s, s + S, ... (padding loads past the last) and one
  // instruction of scales (s < sb_dma) or biases (s - sb_dma < sb_dma), or a padding load
  static constexpr int code_per_wave = (code_dma + S - 1) / S;
  static constexpr int dma_per_wave = code_per_wave + 1;
  // unit buffers: as many as fit (up to 4); slice partials [S][MB][64 lanes][4], two of them
  // when a unit's sums and stores wait until the next unit's barrier (deferred: needs 3
  // unit buffers, since a unit buffer is then refilled two steps after it was read)
  static constexpr int red_bytes = kSlices * MB * 64 * 16;
  static constexpr int nbuf_of(int reds) {
    return (160 * 1024 - reds * red_bytes - 1024) / buf_bytes < 4 ? (160 * 1024 - reds * red_bytes - 1024) / buf_bytes : 4;
  }
  static constexpr bool deferred = QMM_BMV_DEFER && nbuf_of(2) >= 3;
  static constexpr int nbuf = nbuf_of(deferred ? 2 : 1);
  static constexpr int lookahead = deferred ? nbuf - 2 : nbuf - 1;  // units in flight ahead
  static constexpr int red_off = nbuf * buf_bytes;
  static constexpr int dump_off = red_off + (deferred ? 2 : 1) * red_bytes;  // target of padding loads
  static constexpr int lds_bytes = dump_off + 1024;
  static_assert(2 * sb_dma <= kSlices, "one scale or bias instruction per wave");
  static_assert(code_bytes % 1024 == 0, "a unit's codes are whole KB");
  static_assert(nbuf >= 2 && lds_bytes <= 160 * 1024, "LDS");
};

// Global row of LDS row r of unit u (past the end: the last real row, never stored).
// 32-bit: the codes of a weight are below 4 GiB, so every row index and offset fits.
// Rotary QKV: unit u is pairs 8u .. 8u+7, which (head_dim and rot multiples of 16) share
// one head and one region, so their first rows are ra0 .. ra0+7 and their partners
// rb0 .. rb0+7 (ra0, rb0 of pair 8u, passed in as `I` and `rows`).
template <int EPI>
__device__ __forceinline__ uint32_t unit_row(uint32_t rows, uint32_t I, uint32_t u, int r) {
  if constexpr (EPI == EPI_ROPE) {
    return r < 8 ? I + uint32_t(r) : rows + uint32_t(r - 8);
  } else if constexpr (EPI == EPI_SWIGLU) {
    const uint32_t p = min(u * (kUnit / 2) + uint32_t(r & 7), I - 1);
    return r < 8 ? p : I + p;
  } else {
    return min(u * kUnit + uint32_t(r), rows - 1);
  }
}

// Wait until at most N of this wave's vector-memory loads are outstanding and its LDS
// operations are done, then meet the other waves (one asm block: the compiler's own
// barrier would also wait for the unit requested ahead).
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with N = ahead * PER (ahead < 4, block-uniform).
template <int PER>
__device__ __forceinline__ void wait_units_barrier(int ahead) {
  switch (ahead) {
    case 0: wait_loads_barrier<0>(); break;
    case 1: wait_loads_barrier<PER>(); break;
    case 2: wait_loads_barrier<2 * PER>(); break;
    default: wait_loads_barrier<3 * PER>(); break;
  }
}

template <int S, int GPS, int MB, int EPI>
__global__ void __launch_bounds__(64 * S, 1) bmv_u4_kernel(GemvArgs a, int64_t M, int64_t units) {
  using L = Layout<S, GPS, MB>;
  constexpr int R = kRows * MB;  // activation rows per block
  constexpr int K = L::K;
  constexpr int kSlices = S;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::lds_bytes];

  const int lane = threadIdx.x & 63;
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // K slice of this wave
  const int col = lane & 15;  // MFMA column: LDS row of the unit
  const int kb = lane >> 4;   // 8-input block of the MFMA's 32 inputs
  const int64_t mb = blockIdx.y;
  const int64_t rows_here = M - mb * R < R ? M - mb * R : R;
  const uint64_t nrows = uint64_t(a.rows);
  const uint32_t rows32 = uint32_t(a.rows), I32 = uint32_t(a.I);

  const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.codes, nrows * uint64_t(L::row_bytes));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales, nrows * uint64_t(L::sb_row));
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.biases, nrows * uint64_t(L::sb_row));

  // ---- unit -> LDS ------------------------------------------------------------------
  // Code instruction i = S t + s (lane L: byte 1024 i + 16 L of the unit's codes, i.e. row
  // r, slot c) reads chunk c ^ (r & 15) of row r; the row and the in-row byte offset of
  // each of the wave's instructions are fixed for the kernel.  Padding loads (i past the
  // unit's codes, or no scale/bias instruction for this wave) use an offset past the
  // descriptors' ranges, so they read nothing, and land in a dump area of LDS.
  int crow[L::code_per_wave];
  uint32_t cofs[L::code_per_wave];
#pragma unroll
  for (int t = 0; t < L::code_per_wave; ++t) {
    const uint32_t o = 1024u * uint32_t(t * kSlices + s) + 16u * uint32_t(lane);
    const int r = int(o / L::row_bytes);
    const uint32_t c = (o % L::row_bytes) / 16u;
    crow[t] = r < kUnit ? r : 0;  // past the unit's codes: a padding load
    cofs[t] = 16u * (c ^ uint32_t(r & 15));
  }
  // scale/bias instruction of this wave: region byte 1024 j + 16 L
  const bool sb_bias = s >= L::sb_dma;
  const int sb_j = sb_bias ? s - L::sb_dma : s;
  const bool sb_any = s < 2 * L::sb_dma;
  const uint32_t sb_o = 1024u * uint32_t(sb_j) + 16u * uint32_t(lane);
  const int sb_r = int(sb_o / L::sb_row);
  const uint32_t sb_in = sb_o % L::sb_row;
  const __amdgpu_buffer_rsrc_t sbr = sb_bias ? br : sr;
  auto request = [&](int64_t u, int buf) {
    uint8_t* base = lds + buf * L::buf_bytes;
    uint32_t rows_arg = rows32, i_arg = I32;
    if constexpr (EPI == EPI_ROPE) {
      const RopePair rp = rope_pair(uint32_t(u) * 8u, a.rope);  // block-uniform
      i_arg = uint32_t(rp.ra);
      rows_arg = uint32_t(rp.rb);
    }
#pragma unroll
    for (int t = 0; t < L::code_per_wave; ++t) {
      const int i = t * kSlices + s;  // wave-uniform
      const bool real = L::code_dma % kSlices == 0 || i < L::code_dma;
      const uint32_t off = real ? unit_row<EPI>(rows_arg, i_arg, uint32_t(u), crow[t]) * uint32_t(L::row_bytes) + cofs[t]
                                : 0xFFFFFFF0u;
      uint8_t* dst = real ? base + 1024 * i : lds + L::dump_off;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
    }
    // past the scales (padding of the region) or no instruction for this wave: a load
    // beyond every buffer returns zero
    const uint32_t off = sb_any && sb_o < uint32_t(L::sb_bytes)
                             ? unit_row<EPI>(rows_arg, i_arg, uint32_t(u), sb_r) * uint32_t(L::sb_row) + sb_in
                             : 0xFFFFFFF0u;
    uint8_t* dst = sb_any ? base + L::code_bytes + (sb_bias ? L::sb_pad : 0) + 1024 * sb_j : lds + L::dump_off;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sbr, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
  };

  if (int64_t(blockIdx.x) >= units) return;
  const int64_t stride = gridDim.x;
  {
    int64_t u = blockIdx.x;
    // the block's units j = 0, 1, ... (unit u + j * stride) live in buffer j % nbuf; units
    // 0 .. lookahead - 1 are requested here, unit j + lookahead at step j
#pragma unroll
    for (int b = 0; b < L::lookahead; ++b)
      if (u + b * stride < units) request(u + b * stride, b);

    // ---- activations of this slice: MFMA operands, permuted to the nibble-pair order ----
    // Operand lane (row m = lane % 16 of tile t, block kb) of group g, MFMA h holds inputs
    // 64 G + 16 kb + 8 h .. +7 with G = s*GPS + g: the 8 codes its column's lane decodes
    // from code word h of that lane's 16 codes.
    bf16x8_t xa[MB][GPS][2];
    {
      // byte offset of block row m's activations (rows past the block's: past the buffer,
      // read as zeros)
      const uint16_t* xb = a.x + mb * R * K;
      const __amdgpu_buffer_rsrc_t xr = make_rsrc(xb, uint64_t(rows_here) * K * 2);
      uint32_t xrow[MB];
#pragma unroll
      for (int t = 0; t < MB; ++t) xrow[t] = uint32_t(kRows * t + col) * uint32_t(K) * 2u;
#pragma unroll
      for (int t = 0; t < MB; ++t)
#pragma unroll
        for (int g = 0; g < GPS; ++g)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t k0 = uint32_t(64 * (s * GPS + g) + 16 * kb + 8 * h);
            const uint32_t off = xrow[t] == 0xFFFFFFF0u ? xrow[t] : xrow[t] + k0 * 2u;
            const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            const u32x4_t p = {__builtin_amdgcn_perm(d[2], d[0], 0x05040100u), __builtin_amdgcn_perm(d[2], d[0], 0x07060302u),
                               __builtin_amdgcn_perm(d[3], d[1], 0x05040100u), __builtin_amdgcn_perm(d[3], d[1], 0x07060302u)};
            xa[t][g][h] = __builtin_bit_cast(bf16x8_t, p);
          }
    }
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    // xs[r] = sum of group g's 64 inputs of row 4 kb + r of tile t (the MFMA against ones
    // puts that row's sum in every column): kept in registers where they fit (one tile
    // and K <= 5120, two tiles and K <= 3072), else recomputed per unit (the same two
    // MFMAs, so the same values)
    constexpr bool kXsKept = GPS * MB <= 12 && GPS <= 10;
    auto group_xs = [&](int t, int g) {
      const f32x4_t v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[t][g][0], ones, f32x4_t{}, 0, 0, 0);
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[t][g][1], ones, v, 0, 0, 0);
    };
    f32x4_t xs_kept[kXsKept ? MB : 1][kXsKept ? GPS : 1];
    if constexpr (kXsKept) {
#pragma unroll
      for (int t = 0; t < MB; ++t)
#pragma unroll
        for (int g = 0; g < GPS; ++g) xs_kept[t][g] = group_xs(t, g);
    }
    const uint32_t magic = in_vgpr(kMagicPair);
    float* red = reinterpret_cast<float*>(lds + L::red_off);

    // sums of the S slice partials in slice order and the epilogue of unit uu, each output
    // by one lane of one of the waves; rb[j][t][l][r] is slice j's partial of activation row
    // 16 t + 4 (l / 16) + r, column l % 16
    // output row of block row mr
    auto out_row = [&](int mr) -> int64_t { return mb * R + mr; };
    auto epilogue = [&](int64_t uu, const float* rb) {
      auto slice_sum = [&](int t, int l, int r) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < kSlices; ++j) v += rb[((j * MB + t) * 64 + l) * 4 + r];
        return v;
      };
      if constexpr (EPI == EPI_ROPE) {
        // like SwiGLU below: the 8 first rows of the unit's pairs and their partners 8
        // columns further; each pair of each row is rotated by the row's position and
        // stored into its head
        if (lane < 128 * MB / kSlices) {
          const int o = (128 * MB / kSlices) * s + lane;
          const int t = o >> 7, g = (o & 127) >> 2, r = o & 3;
          const int l = (g & 7) + 16 * (g >> 3);
          const int mr = kRows * t + 4 * (l >> 4) + r;
          if (mr < rows_here) {
            const int64_t m = mb * R + mr;  // (no gathered rotary path)
            RopePair rp = rope_pair(uint32_t(uu) * 8u, a.rope);
            const int e = l & 15;  // pair 8 uu + e
            rp.ra += e;
            rp.rb += e;
            rp.da += e;
            rp.db += e;
            if (rp.ri >= 0) rp.ri += e;
            float va = slice_sum(t, l, r), vb = slice_sum(t, l + 8, r);
            if (a.lin_bias) {
              va += bf16_bits_to_f32(a.lin_bias[rp.ra]);
              vb += bf16_bits_to_f32(a.lin_bias[rp.rb]);
            }
            rope_store(a.rope, a.out0, a.out1, a.out2, rp, m, va, vb, a.f32_out);
          }
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
        // 8 gate columns x R rows = 128 MB outputs, 128 MB / S per wave: output o of tile
        // t = o / 128 is gate column g % 8 of block g / 8 (g = (o % 128) / 4) at r = o % 4,
        // with its up column 8 further
        if (lane < 128 * MB / kSlices) {
          const int o = (128 * MB / kSlices) * s + lane;
          const int t = o >> 7, g = (o & 127) >> 2, r = o & 3;
          const int l = (g & 7) + 16 * (g >> 3);
          const int mr = kRows * t + 4 * (l >> 4) + r;  // row within the block
          const int64_t p = uu * (kUnit / 2) + (l & 15);
          if (mr < rows_here && p < a.I)
            store_out(a.out0, out_row(mr) * a.n_out + p, silu_times(slice_sum(t, l, r), slice_sum(t, l + 8, r)),
                      a.f32_out);
        }
      } else {
        // 16 columns x R rows = 256 MB outputs, 256 MB / S per wave: output o of tile
        // t = o / 256 is partial lane (o % 256) / 4 at r = o % 4
        if (lane < 256 * MB / kSlices) {
          const int o = (256 * MB / kSlices) * s + lane;
          const int t = o >> 8, l = (o & 255) >> 2, r = o & 3;
          const int mr = kRows * t + 4 * (l >> 4) + r;
          const int64_t n = uu * kUnit + (l & 15);
          if (mr < rows_here && n < a.rows) {
            const int64_t m = out_row(mr);
            float v = slice_sum(t, l, r);
            if (a.lin_bias) v += bf16_bits_to_f32(a.lin_bias[n]);
            if constexpr (EPI == EPI_QKV) {
              if (n < a.q_out) {
                store_out(a.out0, m * a.q_out + n, v, a.f32_out);
              } else if (n < a.q_out + a.kv_out) {
                store_out(a.out1, m * a.kv_out + (n - a.q_out), v, a.f32_out);
              } else {
                store_out(a.out2, m * a.kv_out + (n - a.q_out - a.kv_out), v, a.f32_out);
              }
            } else {
              store_out(a.out0, m * a.n_out + n, v, a.f32_out);
            }
          }
        }
      }
    };

    int it = 0;
    for (;; ++it) {
      const int buf = it % L::nbuf;
      // request unit it + lookahead, then wait for unit it (the later units' loads may stay
      // in flight); buffer (it + lookahead) % nbuf held unit it - 1 (without deferral: every
      // wave has passed the barrier after reading it) or unit it - 2 (deferred: read before
      // the last barrier)
      const int64_t ua = u + L::lookahead * stride;
      if (ua < units) request(ua, (it + L::lookahead) % L::nbuf);
      const int64_t later = (units - 1 - u) / stride;  // units after u for this block
      wait_units_barrier<L::dma_per_wave>(int(later < L::lookahead ? later : L::lookahead));
      if constexpr (L::deferred) {
        if (it > 0) epilogue(u - stride, red + ((it - 1) & 1) * (L::red_bytes / 4));
      }

      // ---- this wave's slice of unit u ----------------------------------------------------
      const uint8_t* bb = lds + buf * L::buf_bytes;
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(bb + L::code_bytes) + col * (L::sb_row / 2);
      const uint16_t* bi = reinterpret_cast<const uint16_t*>(bb + L::code_bytes + L::sb_pad) + col * (L::sb_row / 2);
      f32x4_t y[MB] = {};
#pragma unroll
      for (int g = 0; g < GPS; ++g) {
        const int G = s * GPS + g;
        // codes 16 kb .. 16 kb + 15 of group G of this lane's column: half (kb & 1) of chunk
        // 2G + kb/2
        const uint32_t c = uint32_t(2 * G + (kb >> 1));
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(bb + col * L::row_bytes + 16 * (c ^ uint32_t(col)) + 8 * (kb & 1));
        const float sv = bf16_bits_to_f32(sc[G]);
        const float bv = bf16_bits_to_f32(bi[G]);
        u32x4_t q[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          q[h] = u32x4_t{nib_pair(w[h], 0, magic), nib_pair(w[h], 1, magic), nib_pair(w[h], 2, magic),
                         nib_pair(w[h], 3, magic)};
#pragma unroll
        for (int t = 0; t < MB; ++t) {
          f32x4_t xs;
          if constexpr (kXsKept) xs = xs_kept[t][g];
          else xs = group_xs(t, g);
          f32x4_t d = {};
#pragma unroll
          for (int h = 0; h < 2; ++h)
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[t][g][h], __builtin_bit_cast(bf16x8_t, q[h]), d, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float dq = fmaf(-128.0f, xs[r], d[r]);  // sum x q (exact 0 for all-zero codes)
            y[t][r] = fmaf(sv, dq, y[t][r]);
            y[t][r] = fmaf(bv, xs[r], y[t][r]);
          }
        }
      }
      if constexpr (L::deferred) {
        // partials of this unit into red buffer it & 1; summed and stored after the next
        // step's barrier (or after the loop)
#pragma unroll
        for (int t = 0; t < MB; ++t)
          *reinterpret_cast<f32x4_t*>(red + (it & 1) * (L::red_bytes / 4) + ((s * MB + t) * 64 + lane) * 4) = y[t];
      } else {
#pragma unroll
        for (int t = 0; t < MB; ++t) *reinterpret_cast<f32x4_t*>(red + ((s * MB + t) * 64 + lane) * 4) = y[t];
        __syncthreads();
        epilogue(u, red);
      }
      u += stride;
      if (u >= units) break;
    }
    if constexpr (L::deferred) {
      __syncthreads();
      epilogue(u - stride, red + (it & 1) * (L::red_bytes / 4));
    }
  }
}

// Instantiated: 8 waves per block (16 measured slower: 28.8 against 27.0 us on the 14B
// gate+up at M = 4), K = 512 * GPS; two 16-row tiles per block (MB = 2, one code decode
// for 32 activation rows) where the registers allow it (K <= 5120).
constexpr int kSlicesUsed = 8;
constexpr int kKStep = 64 * kSlicesUsed;  // K is a multiple of this
constexpr int kMaxGpsTwoTiles = 10;
#ifndef QMM_BMV_TWO_TILES
#define QMM_BMV_TWO_TILES 1
#endif
#define QMM_BMV_GPS(X) X(1) X(2) X(4) X(6) X(8) X(10) X(12) X(14) X(16)

// Row tiles per block for M rows at K = 512 * gps.
inline int tiles_for(int64_t M, int64_t gps) {
  return QMM_BMV_TWO_TILES && M > kRows && gps <= kMaxGpsTwoTiles ? 2 : 1;
}

}  // namespace bmv

bool bmv_supports(int epi, const GemvArgs& a, int64_t M) {
  if (a.bits != 4 || a.gshift != 1 || M < 2 || M > kBmvMaxM || a.K % bmv::kKStep) return false;
  if (epi != EPI_LINEAR && epi != EPI_QKV && epi != EPI_SWIGLU && epi != EPI_ROPE) return false;
  // rotary: units of 8 pairs within one head and one region
  if (epi == EPI_ROPE && (a.rope.head_dim % 16 || a.rope.rot % 16)) return false;
  switch (a.K / bmv::kKStep) {
#define QMM_BMV_CASE(G) case G:
    QMM_BMV_GPS(QMM_BMV_CASE)
#undef QMM_BMV_CASE
      return true;
    default:
      return false;
  }
}

// Above 32 rows the kernel runs one pass of 16 or 32 rows per grid row and reads the
// weights once per pass; it is still taken where the prefill GEMM would leave most of the
// GPU idle (a grid of few 256 x 256 tiles, each walking all of K).  Estimates from the
// rates measured on a 256-CU MI355X (14B / 24B shapes), scaled by the device's compute
// units: a 16-row pass streams the weights at ~11.3 KB/us per CU (2.9 TB/s on 256 CUs) and
// takes at least 8 us, a 32-row pass 1.45 times that; a GEMM round of one tile per CU takes
// ~1.5 us per 64-input step.
#ifndef QMM_BMV_FORCE
#define QMM_BMV_FORCE 0
#endif
bool bmv_preferred(int epi, const GemvArgs& a, int64_t M) {
  if (!bmv_supports(epi, a, M) || gemv_two_rows(a.K, M)) return false;
  if (M <= 32 || QMM_BMV_FORCE) return true;
  const int mb = bmv::tiles_for(M, a.K / bmv::kKStep);
  const double wbytes = double(a.rows) * double(a.K) * (0.5 + 4.0 / 64.0);
  const int64_t cus = device_cus();
  const double bytes_per_us = 11328.0 * double(cus);
  const double pass_us = (wbytes / bytes_per_us > 8.0 ? wbytes / bytes_per_us : 8.0) * (mb == 2 ? 1.45 : 1.0);
  const int64_t rows_per_pass = bmv::kRows * mb;
  const double bmv_us = double((M + rows_per_pass - 1) / rows_per_pass) * pass_us;
  const int64_t n_tiles = epi == EPI_SWIGLU  ? (a.I + 127) / 128
                          : epi == EPI_ROPE  ? ((a.rows >> 1) + 127) / 128
                                             : (a.rows + 255) / 256;
  const int64_t rounds = ((M + 255) / 256 * n_tiles + cus - 1) / cus;
  const double gemm_us = double(rounds) * double(a.K / 64) * 1.5;
  return bmv_us < gemm_us;
}

template <int G, int MB>
static void launch_bmv_tiles(int epi, const GemvArgs& a, int64_t M, int64_t units, hipStream_t st) {
  const int64_t cus = device_cus();
  const dim3 grid{unsigned(units < cus ? units : cus), unsigned((M + bmv::kRows * MB - 1) / (bmv::kRows * MB)), 1u};
  const dim3 block{64u * bmv::kSlicesUsed, 1u, 1u};
  if (epi == EPI_LINEAR)
    bmv::bmv_u4_kernel<bmv::kSlicesUsed, G, MB, EPI_LINEAR><<<grid, block, 0, st>>>(a, M, units);
  else if (epi == EPI_QKV)
    bmv::bmv_u4_kernel<bmv::kSlicesUsed, G, MB, EPI_QKV><<<grid, block, 0, st>>>(a, M, units);
  else if (epi == EPI_ROPE)
    bmv::bmv_u4_kernel<bmv::kSlicesUsed, G, MB, EPI_ROPE><<<grid, block, 0, st>>>(a, M, units);
  else
    bmv::bmv_u4_kernel<bmv::kSlicesUsed, G, MB, EPI_SWIGLU><<<grid, block, 0, st>>>(a, M, units);
}

int launch_bmv(int epi, const GemvArgs& a, int64_t M, hipStream_t st) {
  if (!bmv_supports(epi, a, M)) return 2;
  // SwiGLU: 8 gate/up pairs per unit; rotary QKV: 8 rotating pairs (rows/2 is a multiple
  // of 8 here); otherwise 16 rows
  const int64_t units = epi == EPI_SWIGLU ? (a.I + bmv::kUnit / 2 - 1) / (bmv::kUnit / 2)
                        : epi == EPI_ROPE ? (a.rows >> 1) / (bmv::kUnit / 2)
                                          : (a.rows + bmv::kUnit - 1) / bmv::kUnit;
  const int64_t gps = a.K / bmv::kKStep;
  const bool two = bmv::tiles_for(M, gps) == 2;
  switch (gps) {
#define QMM_BMV_CASE(G)                                                               \
  case G:                                                                             \
    if constexpr (G <= bmv::kMaxGpsTwoTiles) {                                        \
      if (two) {                                                                      \
        launch_bmv_tiles<G, 2>(epi, a, M, units, st);                                 \
        break;                                                                        \
      }                                                                               \
    }                                                                                 \
    launch_bmv_tiles<G, 1>(epi, a, M, units, st);                                     \
    break;
    QMM_BMV_GPS(QMM_BMV_CASE)
#undef QMM_BMV_CASE
    default:
      return 2;
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace qmm
