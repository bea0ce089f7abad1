// Decode (M = 1) kernels for the u4 group-64 affine quantized projections on gfx950.
//
// What is computed: y[n] = sum_k x[k] * (s[n, k/64] * q[n, k] + b[n, k/64]) over the
// rows of a row-concatenated weight, with the fused-QKV split and the SwiGLU
// epilogue of "The Cathedral Doubled Itself" (the two fusions: one quantized
// matmul over [q_out + 2*kv_out, hidden/8], and the same for gate+up before
// SiLU*multiply), and the routed-expert gather over an in-place expert grid
// ("Four Candles for the Cathedral", what's not in this batch: experts are never
// concatenated or copied).  Decode is weight-bandwidth bound ("The Cathedral
// Doubled Itself", what 50 tok/s looks like; "The Canary and the Thread-Local
// Stream", the flat A/B), so every kernel here is built to stream the packed codes
// once from HBM with 16-byte loads.
//
// Layout of the work (one wavefront = 64 lanes):
//   * a row slot is LPR lanes (16 or 32); a wave holds 64/LPR slots, i.e. that many
//     rows at once;
//   * lane i of a slot owns the 32-code chunks i, i+LPR, ..., i+(CPL-1)*LPR of the
//     slot's K slice, so each load instruction of a slot reads LPR*16 contiguous bytes
//     of one row;
//   * the activations of a lane's chunks stay in registers (permuted once to the
//     nibble-pair order) together with their fp32 chunk sums;
//   * per chunk: four code words become exact bf16 pairs (128+q) with one and-or (plus
//     one shift), v_dot2_f32_bf16 accumulates sum x*(128+q) in fp32, and the group's
//     scale and bias enter as  acc += s * (D - 128*xs) + b * xs  (the bias term of
//     w = s*q + b reduces to b times the chunk's activation sum);
//   * lanes of a slot are summed with DPP; when K is split across waves (ksplit > 1)
//     the per-wave partials meet in LDS and are added in wave order.
// The reduction order of a row depends only on K, never on the row index or on the
// number of rows in the call.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_rope.h"

#ifndef QMM_BITS
#define QMM_BITS 4
#endif

namespace qmm {
// Each code width is its own object (this file built once per width with -DQMM_BITS=N):
// its kernels and launchers live in namespace qmm::b<N>.
namespace QMM_BITS_NS {

constexpr int kBits = QMM_BITS;  // storage bits per code
#if QMM_FP8
static_assert(QMM_BITS == 8, "fp8 codes are 8 bits");
using Cd = CodecE4M3;
#else
using Cd = Codec<kBits>;
#endif
constexpr int kChunkBytes = 4 * kBits;  // 32 codes
constexpr int kMaxCplSplit16 = (kBits == 2 || kBits == 4) ? 4 : 3;


// Activations of this lane's chunks, in registers for the whole kernel, read through a
// buffer descriptor bounded by K: a chunk past the end of the K slice (ragged K) reads
// zeros, so it contributes exactly nothing whatever codes, scale and bias sit there.
template <int LPR, int CPL>
__device__ __forceinline__ void load_x_chunks(__amdgpu_buffer_rsrc_t xr, uint32_t c0, uint32_t xp[CPL][16],
                                              float xs[CPL]) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint32_t off = (c0 + uint32_t(LPR * i)) * 64u;
    uint32_t d[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16u * v, 0, 0);
      d[4 * v + 0] = t[0];
      d[4 * v + 1] = t[1];
      d[4 * v + 2] = t[2];
      d[4 * v + 3] = t[3];
    }
    Cd::permute(d, xp[i]);
    xs[i] = chunk_xsum(xp[i]);
  }
}

// The packed codes and the group scales/biases of one row for this lane's chunks.
template <int CPL>
struct RowData {
  uint32_t w[CPL][kBits];
  uint16_t s[CPL], b[CPL];
};

// The kBits words of one chunk at byte `off` (16-, 12- or 8-byte loads).
__device__ __forceinline__ void load_chunk(uint32_t (&w)[kBits], __amdgpu_buffer_rsrc_t cr, uint32_t off) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
  int i = 0;
#pragma unroll
  for (; i + 4 <= kBits; i += 4) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(cr, off + 4u * i, 0, kLoadNT);
    w[i] = v[0];
    w[i + 1] = v[1];
    w[i + 2] = v[2];
    w[i + 3] = v[3];
  }
  if constexpr (kBits % 4 == 3) {
    const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(cr, off + 4u * i, 0, kLoadNT);
    w[i] = v[0];
    w[i + 1] = v[1];
    w[i + 2] = v[2];
  } else if constexpr (kBits % 4 == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(cr, off + 4u * i, 0, kLoadNT);
    w[i] = v[0];
    w[i + 1] = v[1];
  }
}

// Chunk c0 + LPR*i of row `row`: codes at byte row*K*bits/8 + 4*bits*c, scale/bias of
// group c >> gshift (group size 32 << gshift) at 2*(row*K/G + (c >> gshift)); consecutive
// chunks of a lane are LPR*4*bits (codes) and 2*(LPR >> gshift) (groups) bytes apart.
template <int LPR, int CPL>
__device__ __forceinline__ void load_row(RowData<CPL>& r, __amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr,
                                         __amdgpu_buffer_rsrc_t br, uint32_t row, uint32_t row_bytes,
                                         uint32_t row_groups, uint32_t c0, int gshift) {
  const uint32_t co = row * row_bytes + c0 * uint32_t(kChunkBytes);
  const uint32_t go = (row * row_groups + (c0 >> gshift)) * 2u;
  const uint32_t gstep = uint32_t(LPR >> gshift) * 2u;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    load_chunk(r.w[i], cr, co + uint32_t(i * LPR * kChunkBytes));
    r.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, go + uint32_t(i) * gstep, 0, 0);
    r.b[i] = __builtin_amdgcn_raw_buffer_load_b16(br, go + uint32_t(i) * gstep, 0, 0);
  }
}

// Partial dot product of one row over this lane's chunks (fp32).
template <int CPL>
__device__ __forceinline__ float row_partial(const RowData<CPL>& r, const uint32_t xp[CPL][16], const float xs[CPL],
                                             uint32_t magic) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const float d = Cd::dot_q(r.w[i], xp[i], xs[i], magic);  // sum x q over the chunk
    acc = fmaf(bf16_bits_to_f32(r.s[i]), d, acc);
    acc = fmaf(bf16_bits_to_f32(r.b[i]), xs[i], acc);
  }
  return acc;
}

// Row of the weight handled by slot `slot` of unit `unit`, and whether it exists.  The
// paired epilogues (SwiGLU, rotary QKV) put the two rows of a pair in slots s and s + P,
// 32 lanes apart.
template <int LPR, int EPI>
__device__ __forceinline__ int64_t unit_row(int64_t unit, int slot, const GemvArgs& a, bool* valid) {
  constexpr int RPI = 64 / LPR;
  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int P = RPI / 2;
    const int64_t pair = unit * P + (slot % P);
    *valid = pair < a.I;
    const int64_t r = slot < P ? pair : a.I + pair;
    return *valid ? r : 0;
  } else if constexpr (EPI == EPI_ROPE) {
    constexpr int P = RPI / 2;
    const int64_t pair = unit * P + (slot % P);
    *valid = pair < (a.rows >> 1);
    const RopePair rp = rope_pair(uint32_t(*valid ? pair : 0), a.rope);
    return slot < P ? rp.ra : rp.rb;
  } else {
    const int64_t r = unit * RPI + slot;
    *valid = r < a.rows;
    return *valid ? r : (a.rows - 1);
  }
}

// Operands of a unit's epilogue that come from memory, fetched together with the unit's
// rows so that its store does not wait on a dependent load: the rotary cos/sin of the
// lane's pair (EPI_ROPE; `trow` is the token's table row).  Nothing for the others.
struct EpiPre {
  float c, s;
};
template <int LPR, int EPI>
__device__ __forceinline__ const float* epi_table_row(const GemvArgs& a, int64_t m) {
  if constexpr (EPI == EPI_ROPE) {
    const int32_t pos = min(max(a.rope.positions[m], 0), a.rope.max_pos - 1);
    return a.rope.cos_sin + int64_t(pos) * a.rope.rot;
  } else {
    return nullptr;
  }
}
template <int LPR, int EPI>
__device__ __forceinline__ void epi_fetch(EpiPre& p, int64_t u, int slot, const GemvArgs& a, const float* trow) {
  if constexpr (EPI == EPI_ROPE) {
    constexpr int P = (64 / LPR) / 2;
    const int64_t pair = u * P + (slot % P);
    const RopePair rp = rope_pair(uint32_t(pair < (a.rows >> 1) ? pair : 0), a.rope);
    const int ri = rp.ri >= 0 ? rp.ri : 0;
    p.c = trow[ri];
    p.s = trow[(a.rope.rot >> 1) + ri];
  }
}

// Store of one row unit's result (slot totals after slot_reduce).
template <int LPR, int EPI>
__device__ __forceinline__ void gemv_store(const GemvArgs& a, float v, int64_t u, int slot, int lane,
                                           int64_t out_base, const EpiPre& ep, int64_t m) {
  constexpr int RPI = 64 / LPR;
  constexpr int P = RPI / 2;
  bool valid;
  const int64_t r = unit_row<LPR, EPI>(u, slot, a, &valid);
  if constexpr (EPI == EPI_SWIGLU) {
    const float up = __shfl_xor(v, 32);
    if (valid && slot < P && lane == slot_result_lane<LPR>(slot))
      store_out(a.out0, out_base + u * P + slot, silu_times(v, up), a.f32_out);
  } else if constexpr (EPI == EPI_ROPE) {
    if (valid && a.lin_bias) v += bf16_bits_to_f32(a.lin_bias[r]);
    const float vb = __shfl_xor(v, 32);
    if (valid && slot < P && lane == slot_result_lane<LPR>(slot))
      rope_store_cs(a.rope, a.out0, a.out1, a.out2, rope_pair(uint32_t(u * P + slot), a.rope), m, v, vb,
                    ep.c, ep.s, a.f32_out);
  } else {
    if (valid && lane == slot_result_lane<LPR>(slot)) {
      if (a.lin_bias) v += bf16_bits_to_f32(a.lin_bias[r]);
      if constexpr (EPI == EPI_QKV) {
        if (r < a.q_out) {
          store_out(a.out0, m * a.q_out + r, v, a.f32_out);
        } else if (r < a.q_out + a.kv_out) {
          store_out(a.out1, m * a.kv_out + (r - a.q_out), v, a.f32_out);
        } else {
          store_out(a.out2, m * a.kv_out + (r - a.q_out - a.kv_out), v, a.f32_out);
        }
      } else {
        store_out(a.out0, out_base + r, v, a.f32_out);
      }
    }
  }
}

// ---- K-split decode kernel (ksplit 8 or 16: 5120 < K <= 65536) -------------------------
// A block is one row group of KS waves; wave ks owns the K slice [ks*LPR*CPL*32, ...) of
// every row the group handles.  After each row unit the KS partial sums meet in LDS and
// wave 0 adds them in wave order and stores; the barrier this takes also keeps the waves
// on the same rows at the same time (each unit's rows are then read as one contiguous
// stretch per row), which measured faster than reducing once at the end.  The units are
// spread evenly over the row groups.
#ifndef QMM_GEMV_DEPTH
#define QMM_GEMV_DEPTH 1
#endif
#ifndef QMM_GEMV_WAVES_PER_CU
#define QMM_GEMV_WAVES_PER_CU 8
#endif

template <int LPR, int CPL, int KS, int EPI, bool MOE, int DEPTH = QMM_GEMV_DEPTH>
__global__ void __launch_bounds__(64 * KS) gemv_u4_kernel(GemvArgs a, int64_t per_group, int64_t extra) {
  constexpr int RPI = 64 / LPR;
  constexpr int P = RPI / 2;
  static_assert(KS > 1, "the single-slice kernel handles ksplit 1");
  __shared__ float red[2][KS][RPI];

  const int lane = threadIdx.x & 63;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane / LPR;
  const int li = lane % LPR;
  const int64_t words = (a.K * kBits) >> 5;
  const int64_t groups = a.K >> (5 + a.gshift);
  const int64_t gi = blockIdx.x;
  const int64_t u_begin = gi * per_group + (gi < extra ? gi : extra);
  const int64_t u_end = u_begin + per_group + (gi < extra ? 1 : 0);

  const uint32_t* codes = a.codes;
  const uint16_t* scales = a.scales;
  const uint16_t* biases = a.biases;
  const uint16_t* x = a.x;
  int64_t out_base;
  if constexpr (MOE) {
    // blockIdx.y is the routed slot k; its expert's rows are read in place from the grid,
    // its activation row is k / moe_div (several tokens) or the one row.
    const int k = blockIdx.y;
    const int32_t e = a.expert_ids[k];
    out_base = int64_t(k) * a.I;
    if (a.moe_div > 0) x += (int64_t(k) / a.moe_div) * a.K;
    if (e < 0 || e >= a.E) {
      // no expert: this slot's h is zero
      if (ks == 0) {
        for (int64_t u = u_begin; u < u_end; ++u) {
          bool valid;
          (void)unit_row<LPR, EPI>(u, slot, a, &valid);
          if (valid && slot < P && lane == slot_result_lane<LPR>(slot))
            store_out(a.out0, out_base + u * P + slot, 0.f, a.f32_out);
        }
      }
      return;
    }
    const int64_t off = int64_t(e) * a.rows;
    codes += off * words;
    scales += off * groups;
    biases += off * groups;
  } else {
    x += int64_t(blockIdx.y) * a.K;
    out_base = int64_t(blockIdx.y) * a.n_out;
  }

  const uint32_t row_bytes = uint32_t((a.K * kBits) >> 3);
  const uint32_t row_groups = uint32_t(groups);
  const uint64_t nrows = uint64_t(a.rows);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(codes, nrows * row_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, nrows * row_groups * 2);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(biases, nrows * row_groups * 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, uint64_t(a.K) * 2);
  const uint32_t c0 = uint32_t(ks * (LPR * CPL) + li);

  uint32_t xp[CPL][16];
  float xs[CPL];
  const uint32_t magic = in_vgpr(kMagicPair);

  // Ring of DEPTH row buffers: unit u is computed from buf[(u - u_begin) % DEPTH], and
  // the buffer is refilled with unit u + DEPTH right after.
  RowData<CPL> buf[DEPTH];
  EpiPre ep[DEPTH];
  const float* trow = epi_table_row<LPR, EPI>(a, blockIdx.y);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (u_begin + d < u_end) {
      bool valid;
      const int64_t row = unit_row<LPR, EPI>(u_begin + d, slot, a, &valid);
      load_row<LPR, CPL>(buf[d], cr, sr, br, uint32_t(row), row_bytes, row_groups, c0, a.gshift);
      epi_fetch<LPR, EPI>(ep[d], u_begin + d, slot, a, trow);
    }
  }
  load_x_chunks<LPR, CPL>(xr, c0, xp, xs);

  for (int64_t u0 = u_begin; u0 < u_end; u0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t u = u0 + d;
      if (u < u_end) {
        const float v = slot_reduce<LPR>(row_partial<CPL>(buf[d], xp, xs, magic));
        const EpiPre cur = ep[d];
        if (u + DEPTH < u_end) {
          bool valid;
          const int64_t row = unit_row<LPR, EPI>(u + DEPTH, slot, a, &valid);
          load_row<LPR, CPL>(buf[d], cr, sr, br, uint32_t(row), row_bytes, row_groups, c0, a.gshift);
          epi_fetch<LPR, EPI>(ep[d], u + DEPTH, slot, a, trow);
        }
        // double-buffered by unit parity: the next write to this buffer comes after the
        // next unit's barrier, which wave 0 reaches only after reading this one
        float (*rb)[RPI] = red[u & 1];
        if (lane == slot_result_lane<LPR>(slot)) rb[ks][slot] = v;
        __syncthreads();
        if (ks == 0) {
          float t = 0.f;
#pragma unroll
          for (int j = 0; j < KS; ++j) t += rb[j][slot];
          gemv_store<LPR, EPI>(a, t, u, slot, lane, out_base, cur, blockIdx.y);
        }
      }
    }
  }
}

// ---- single-slice decode kernel (ksplit == 1: K <= 5120) --------------------------------
// The same per-row arithmetic and reduction order as gemv_u4_kernel (results are bit for
// bit the same), but the activations, which every wave needs in full, are staged once
// per block in LDS: each 32-code chunk permuted to the nibble-pair order, with its chunk
// sum.  A wave then reads its chunks from LDS instead of issuing its own global loads
// (the two row slots of a wave used to fetch the same activations), and its first row
// units' codes are already in flight while the block stages them.
constexpr int kXStride = 20;  // words per staged activation chunk (16 + 4 padding)
constexpr int kWavesS1 = 4;   // waves (row groups) per block

template <int LPR, int CPL>
struct S1Layout {
  static constexpr int RPI = 64 / LPR;
  static constexpr int C = LPR * CPL;                // chunks a row slot covers
  static constexpr int x_words = C * kXStride + C;  // permuted activations, then chunk sums
  static constexpr size_t lds_bytes() { return size_t(x_words) * 4; }
};


#ifndef QMM_S1_DEPTH
#define QMM_S1_DEPTH 1
#endif
#ifndef QMM_S1_WAVES_PER_CU
#define QMM_S1_WAVES_PER_CU 12  // fallback if the occupancy query fails
#endif
// NR activation rows per block (two: both rows' results from one read of the weights,
// each row computed exactly as alone); the first row's activations stay in registers,
// the second's are read from the block's LDS copy per row unit.
// The body of the single-slice kernel for block (bx, by) of a grid of WPB-wave blocks (0:
// blockDim.x / 64), shared by gemv_u4_s1_kernel and the stage-1 blocks of the one-launch
// MoE layer.
template <int LPR, int CPL, int EPI, bool MOE, int NR, int DEPTH, int WPB>
__device__ __forceinline__ void s1_body(const GemvArgs& a, int64_t per_wave, int64_t extra, uint32_t bx,
                                        uint32_t by, uint32_t* s1_lds) {
  using Lay = S1Layout<LPR, CPL>;
  constexpr int RPI = Lay::RPI;
  constexpr int P = RPI / 2;
  constexpr int C = Lay::C;
  static_assert(NR == 1 || (NR == 2 && !MOE), "two rows: not the routed experts");
  uint32_t* xl = s1_lds;  // row r at s1_lds + r * x_words
  float* xsl = reinterpret_cast<float*>(s1_lds + C * kXStride);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane / LPR;
  const int li = lane % LPR;
  const int64_t words = (a.K * kBits) >> 5;
  const int64_t groups = a.K >> (5 + a.gshift);
  // the units are spread evenly over the waves: every wave takes `per_wave` consecutive
  // units and the first `extra` waves one more
  const int wpb = WPB > 0 ? WPB : int(blockDim.x >> 6);  // WPB = 0: the block's own size
  const int64_t gw = int64_t(bx) * wpb + wave;
  const int64_t u_begin = gw * per_wave + (gw < extra ? gw : extra);
  const int64_t u_end = u_begin + per_wave + (gw < extra ? 1 : 0);

  const uint32_t* codes = a.codes;
  const uint16_t* scales = a.scales;
  const uint16_t* biases = a.biases;
  const uint16_t* x = a.x;
  int64_t out_base;
  if constexpr (MOE) {
    // `by` is the routed slot k (the whole block shares it); its expert's rows are
    // read in place from the grid, its activation row is k / moe_div (several tokens) or
    // the one row.
    const int k = by;
    const int32_t e = a.expert_ids[k];
    out_base = int64_t(k) * a.I;
    if (a.moe_div > 0) x += (int64_t(k) / a.moe_div) * a.K;
    if (e < 0 || e >= a.E) {
      // no expert: this slot's h is zero
      for (int64_t u = u_begin; u < u_end; ++u) {
        bool valid;
        (void)unit_row<LPR, EPI>(u, slot, a, &valid);
        if (valid && slot < P && lane == slot_result_lane<LPR>(slot))
          store_out(a.out0, out_base + u * P + slot, 0.f, a.f32_out);
      }
      return;
    }
    const int64_t off = int64_t(e) * a.rows;
    codes += off * words;
    scales += off * groups;
    biases += off * groups;
  } else {
    x += int64_t(by) * NR * a.K;
    out_base = int64_t(by) * NR * a.n_out;
  }
  const int64_t m0 = int64_t(by) * NR;  // activation row of the block's first row

  const uint32_t row_bytes = uint32_t((a.K * kBits) >> 3);
  const uint64_t nrows = uint64_t(a.rows);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(codes, nrows * row_bytes);
  const uint32_t c0 = uint32_t(li);
  const uint32_t magic = in_vgpr(kMagicPair);
  const uint32_t row_groups = uint32_t(groups);
  const __amdgpu_buffer_rsrc_t sr0 = make_rsrc(scales, nrows * row_groups * 2);
  const __amdgpu_buffer_rsrc_t br0 = make_rsrc(biases, nrows * row_groups * 2);

  // first row units' codes, scales and biases in flight before the staging
  RowData<CPL> buf[DEPTH];
  EpiPre ep[DEPTH], ep1[DEPTH];  // ep1: the second row's (NR = 2)
  const float* trow = epi_table_row<LPR, EPI>(a, m0);
  const float* trow1 = NR == 2 ? epi_table_row<LPR, EPI>(a, m0 + 1) : nullptr;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (u_begin + d < u_end) {
      bool valid;
      const int64_t row = unit_row<LPR, EPI>(u_begin + d, slot, a, &valid);
      load_row<LPR, CPL>(buf[d], cr, sr0, br0, uint32_t(row), row_bytes, row_groups, c0, a.gshift);
      epi_fetch<LPR, EPI>(ep[d], u_begin + d, slot, a, trow);
      if constexpr (NR == 2) epi_fetch<LPR, EPI>(ep1[d], u_begin + d, slot, a, trow1);
    }
  }

  // stage the activations: chunk c (32 of them, zeros past K) permuted, and its sum
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + rr * a.K, uint64_t(a.K) * 2);
    uint32_t* xlr = xl + rr * Lay::x_words;
    float* xslr = xsl + rr * Lay::x_words;
    for (int c = threadIdx.x; c < C; c += 64 * wpb) {
      uint32_t d[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(xr, uint32_t(c) * 64u + 16u * v, 0, 0);
        d[4 * v + 0] = t[0];
        d[4 * v + 1] = t[1];
        d[4 * v + 2] = t[2];
        d[4 * v + 3] = t[3];
      }
      uint32_t xp[16];
      Cd::permute(d, xp);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(xlr + c * kXStride);
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[v] = u32x4_t{xp[4 * v], xp[4 * v + 1], xp[4 * v + 2], xp[4 * v + 3]};
      xslr[c] = chunk_xsum(xp);
    }
  }
  __syncthreads();

  uint32_t xp[CPL][16];
  float xs[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = li + LPR * i;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(xl + c * kXStride);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4_t t = src[v];
      xp[i][4 * v + 0] = t[0];
      xp[i][4 * v + 1] = t[1];
      xp[i][4 * v + 2] = t[2];
      xp[i][4 * v + 3] = t[3];
    }
    xs[i] = xsl[c];
  }
  float xs1[CPL];
  if constexpr (NR == 2) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) xs1[i] = xsl[Lay::x_words + li + LPR * i];
  }

  for (int64_t u0 = u_begin; u0 < u_end; u0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t u = u0 + d;
      if (u < u_end) {
        float v, v1 = 0.f;
        if constexpr (NR == 2) {
          // the sums of row_partial for both rows, chunk by chunk (one decode of the codes
          // serves both), the second row's activations read from LDS per chunk
          float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) {
            // an offset the compiler cannot see through, so that the reads stay here instead
            // of being hoisted out of the loop into 16 * CPL more registers
            uint32_t xo = uint32_t(Lay::x_words + (li + LPR * i) * kXStride);
            asm volatile("" : "+v"(xo));
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(xl + xo);
            uint32_t xq[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4_t t = src[q];
              xq[4 * q + 0] = t[0];
              xq[4 * q + 1] = t[1];
              xq[4 * q + 2] = t[2];
              xq[4 * q + 3] = t[3];
            }
            const float sv = bf16_bits_to_f32(buf[d].s[i]), bv = bf16_bits_to_f32(buf[d].b[i]);
            const float d0 = Cd::dot_q(buf[d].w[i], xp[i], xs[i], magic);
            const float d1 = Cd::dot_q(buf[d].w[i], xq, xs1[i], magic);
            acc0 = fmaf(sv, d0, acc0);
            acc0 = fmaf(bv, xs[i], acc0);
            acc1 = fmaf(sv, d1, acc1);
            acc1 = fmaf(bv, xs1[i], acc1);
          }
          v = slot_reduce<LPR>(acc0);
          v1 = slot_reduce<LPR>(acc1);
        } else {
          v = slot_reduce<LPR>(row_partial<CPL>(buf[d], xp, xs, magic));
        }
        const EpiPre cur = ep[d], cur1 = ep1[d];
        if (u + DEPTH < u_end) {
          bool valid;
          const int64_t row = unit_row<LPR, EPI>(u + DEPTH, slot, a, &valid);
          load_row<LPR, CPL>(buf[d], cr, sr0, br0, uint32_t(row), row_bytes, row_groups, c0, a.gshift);
          epi_fetch<LPR, EPI>(ep[d], u + DEPTH, slot, a, trow);
          if constexpr (NR == 2) epi_fetch<LPR, EPI>(ep1[d], u + DEPTH, slot, a, trow1);
        }
        gemv_store<LPR, EPI>(a, v, u, slot, lane, out_base, cur, m0);
        if constexpr (NR == 2) gemv_store<LPR, EPI>(a, v1, u, slot, lane, out_base + a.n_out, cur1, m0 + 1);
      }
    }
  }
}

#ifndef QMM_S1_MINW
#define QMM_S1_MINW 1
#endif
template <int LPR, int CPL, int EPI, bool MOE, int NR = 1, int DEPTH = QMM_S1_DEPTH>
__global__ void __launch_bounds__(64 * kWavesS1, QMM_S1_MINW) gemv_u4_s1_kernel(GemvArgs a, int64_t per_wave,
                                                                              int64_t extra) {
  extern __shared__ __attribute__((aligned(16))) uint32_t s1_lds[];
  s1_body<LPR, CPL, EPI, MOE, NR, DEPTH, kWavesS1>(a, per_wave, extra, blockIdx.x, blockIdx.y, s1_lds);
}

// Routed-expert stage 2: y[r] = sum_k p_k * (D_{e_k} h_k)[r], for each token (blockIdx.y)
// of its topk slots.  A block's kw waves split
// the routed slots (wave w takes k = w, w+kw, ...) and walk the block's `upw` row units
// for each; every wave adds its slots in increasing k into its own LDS slice, and the
// slices are then added in wave order.  No atomics, so the order is fixed.
constexpr int kMaxUnitsPerCombineBlock = 16;
constexpr int kDownGroup = 4;  // row units whose loads a wave requests together
#ifndef QMM_MOE_DOWN_BLOCKS
#define QMM_MOE_DOWN_BLOCKS 256
#endif

template <int LPR, int CPL>
__global__ void __launch_bounds__(512) moe_down_kernel(GemvArgs a, int64_t units, int upw) {
  constexpr int RPI = 64 / LPR;
  __shared__ float red[8][kMaxUnitsPerCombineBlock][RPI];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kw = blockDim.x >> 6;
  const int slot = lane / LPR;
  const int li = lane % LPR;
  const bool result_lane = lane == slot_result_lane<LPR>(slot);
  const int64_t u_begin = int64_t(blockIdx.x) * upw;
  const int nu = int(u_begin + upw < units ? upw : units - u_begin);
  const uint32_t row_bytes = uint32_t((a.K * kBits) >> 3);
  const uint32_t row_groups = uint32_t(a.K >> (5 + a.gshift));
  const uint64_t expert_words = uint64_t(a.rows) * uint64_t((a.K * kBits) >> 5);
  const uint64_t expert_groups = uint64_t(a.rows) * row_groups;
  const uint32_t c0 = uint32_t(li);
  const uint32_t magic = in_vgpr(kMagicPair);

  if (result_lane)
    for (int u = 0; u < nu; ++u) red[wave][u][slot] = 0.f;

  // blockIdx.y is the token: its slots are pairs token*topk + k of ids, weights and h
  const int64_t pair0 = int64_t(blockIdx.y) * a.topk;
  for (int k = wave; k < a.topk; k += kw) {
    const int32_t e = a.expert_ids[pair0 + k];
    if (e < 0 || e >= a.E) continue;  // no expert: contributes nothing
    const float p = a.expert_w[pair0 + k];
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.codes + uint64_t(e) * expert_words, expert_words * 4);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales + uint64_t(e) * expert_groups, expert_groups * 2);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(a.biases + uint64_t(e) * expert_groups, expert_groups * 2);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x + (pair0 + k) * a.K, uint64_t(a.K) * 2);
    // the units in groups of kDownGroup, every load of a group (and, with the first, the
    // slot's h) requested before any of its arithmetic: one memory round trip per group
    uint32_t xp[CPL][16];
    float xs[CPL];
    for (int g0 = 0; g0 < nu; g0 += kDownGroup) {
      RowData<CPL> buf[kDownGroup];
#pragma unroll
      for (int j = 0; j < kDownGroup; ++j)
        if (g0 + j < nu)
          load_row<LPR, CPL>(buf[j], cr, sr, br, uint32_t((u_begin + g0 + j) * RPI + slot), row_bytes, row_groups,
                             c0, a.gshift);
      if (g0 == 0) load_x_chunks<LPR, CPL>(xr, c0, xp, xs);
#pragma unroll
      for (int j = 0; j < kDownGroup; ++j)
        if (g0 + j < nu) {
          const float v = slot_reduce<LPR>(row_partial<CPL>(buf[j], xp, xs, magic));
          if (result_lane) red[wave][g0 + j][slot] = fmaf(p, v, red[wave][g0 + j][slot]);
        }
    }
  }
  __syncthreads();
  if (wave != 0 || !result_lane) return;
  for (int u = 0; u < nu; ++u) {
    const int64_t r = (u_begin + u) * RPI + slot;
    if (r < a.rows) {
      float v = 0.f;
      for (int j = 0; j < kw; ++j) v += red[j][u][slot];
      store_out(a.out0, int64_t(blockIdx.y) * a.rows + r, v, a.f32_out);
    }
  }
}

bool gemv_shape_for_k(int64_t K, GemvShape* o) {
  if (K < 64 || K % 64) return false;
  const int64_t C = K / 32;
  if (C <= 16) {
    *o = GemvShape{16, 1, 1};
    return true;
  }
  // K slices per row: 1 wave up to K = 5120, 8 waves up to 40960, 16 waves up to 65536;
  // at most 5 chunks (80 activation registers) per lane.
  const int ks = C <= 160 ? 1 : (C <= 1280 ? 8 : 16);
  const int64_t cpl = (C + 32 * ks - 1) / (32 * ks);
  // the 16-way split runs 1024 threads (128 registers each): 3 chunks per lane for the
  // codes that take more than 4 words per chunk or a funnel shift per code pair
  if (cpl > (ks == 16 ? kMaxCplSplit16 : 5)) return false;
  *o = GemvShape{32, int(cpl), ks};
  return true;
}

static int finish_launch() { return hipGetLastError() == hipSuccess ? 0 : 6; }

#define QMM_GEMV_CASE(L, C, K, EPI, MOE)                                                                 \
  case (L * 10000 + C * 100 + K):                                                                        \
    gemv_u4_kernel<L, C, K, EPI, MOE><<<grid, block, 0, s>>>(a, units / upw, units % upw);               \
    break;
#define QMM_GEMV_S1_CASE(L, C, EPI, MOE)                                                              \
  case (L * 10000 + C * 100 + 1): {                                                                  \
    const int64_t w = s1_waves(units, batch, s1_resident_waves<L, C, EPI, MOE>());                  \
    const dim3 g1{unsigned(w / kWavesS1), unsigned(batch), 1u};                                       \
    gemv_u4_s1_kernel<L, C, EPI, MOE>                                                                \
        <<<g1, dim3{64u * kWavesS1, 1u, 1u}, S1Layout<L, C>::lds_bytes(), s>>>(a, units / w, units % w); \
  } break;

// 4 chunks per lane in the 16-way split only where they fit (kMaxCplSplit16)
#if QMM_BITS == 2 || QMM_BITS == 4
#define QMM_GEMV_CASE_SPLIT16_CPL4(EPI, MOE) QMM_GEMV_CASE(32, 4, 16, EPI, MOE)
#else
#define QMM_GEMV_CASE_SPLIT16_CPL4(EPI, MOE)
#endif

#define QMM_GEMV_CASES(EPI, MOE)                                                  \
  switch (sh.lpr * 10000 + sh.cpl * 100 + sh.ksplit) {                            \
    QMM_GEMV_S1_CASE(16, 1, EPI, MOE)                                             \
    QMM_GEMV_S1_CASE(32, 1, EPI, MOE)                                             \
    QMM_GEMV_S1_CASE(32, 2, EPI, MOE)                                             \
    QMM_GEMV_S1_CASE(32, 3, EPI, MOE)                                             \
    QMM_GEMV_S1_CASE(32, 4, EPI, MOE)                                             \
    QMM_GEMV_S1_CASE(32, 5, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 1, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 2, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 3, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 4, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 5, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 3, 16, EPI, MOE)                                            \
    QMM_GEMV_CASE_SPLIT16_CPL4(EPI, MOE)                                          \
    default: return 2;                                                            \
  }

// Grid of the decode kernels.  The row units are spread evenly over the waves of the
// single-slice kernel and over the row groups of the K-split kernel.  The single-slice
// kernel gets as many waves as the GPU holds at once for that instance (its register use
// sets the occupancy; queried once per instance) but never more waves than units; the
// K-split kernel about QMM_GEMV_WAVES_PER_CU waves per compute unit.
static int64_t target_waves() { return int64_t(device_cus()) * QMM_GEMV_WAVES_PER_CU; }

template <int L, int C, int EPI, bool MOE, int NR = 1>
static int64_t s1_resident_waves() {
  static const int64_t blocks_per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, gemv_u4_s1_kernel<L, C, EPI, MOE, NR>, 64 * kWavesS1,
                                                     NR * S1Layout<L, C>::lds_bytes()) != hipSuccess ||
        b < 1)
      b = QMM_S1_WAVES_PER_CU / kWavesS1;
    return int64_t(b);
  }();
  return int64_t(device_cus()) * kWavesS1 * blocks_per_cu;
}

// waves of a single-slice launch per batch entry (a multiple of the block's waves)
static int64_t s1_waves(int64_t units, int64_t batch, int64_t resident) {
  const int64_t want = (resident + batch - 1) / batch;
  int64_t w = want < units ? want : units;
  return (w + kWavesS1 - 1) / kWavesS1 * kWavesS1;
}

static void gemv_geometry(const GemvShape& sh, int epi, const GemvArgs& a, int64_t batch, int64_t* units, int* n,
                          int64_t* blocks, int* threads) {
  const int rpi = 64 / sh.lpr;
  const int64_t pairs = epi == EPI_SWIGLU ? a.I : (a.rows >> 1);
  *units = (epi == EPI_SWIGLU || epi == EPI_ROPE) ? (pairs + rpi / 2 - 1) / (rpi / 2) : (a.rows + rpi - 1) / rpi;
  // K-split kernel (the single-slice cases compute their own grid)
  const int64_t want = (target_waves() / sh.ksplit + batch - 1) / batch;
  const int64_t g = want < *units ? want : *units;
  *n = int(g);
  *blocks = g;
  *threads = 64 * sh.ksplit;
}

// Both rows of an M = 2 call in one single-slice launch (gemv_two_rows).
template <int EPI>
static int launch_s1_two_rows(const GemvShape& sh, const GemvArgs& a, int64_t units, hipStream_t s) {
  switch (sh.lpr * 100 + sh.cpl) {
#define QMM_S1_TWO_ROWS_CASE(L, C)                                                                      \
  case L * 100 + C: {                                                                                   \
    const int64_t w = s1_waves(units, 1, s1_resident_waves<L, C, EPI, false, 2>());                     \
    gemv_u4_s1_kernel<L, C, EPI, false, 2><<<dim3{unsigned(w / kWavesS1), 1u, 1u}, dim3{64u * kWavesS1, 1u, 1u}, \
                                             2 * S1Layout<L, C>::lds_bytes(), s>>>(a, units / w, units % w);    \
  } break;
    QMM_S1_TWO_ROWS_CASE(16, 1)
    QMM_S1_TWO_ROWS_CASE(32, 1)
    QMM_S1_TWO_ROWS_CASE(32, 2)
    QMM_S1_TWO_ROWS_CASE(32, 3)
    QMM_S1_TWO_ROWS_CASE(32, 4)
    QMM_S1_TWO_ROWS_CASE(32, 5)
#undef QMM_S1_TWO_ROWS_CASE
    default:
      return 2;
  }
  return finish_launch();
}

int launch_gemv(int epi, const GemvArgs& a, int64_t M, hipStream_t s) {
  GemvShape sh;
  if (!gemv_shape_for_k(a.K, &sh)) return 2;
  if (gemv_two_rows(a.K, M) && sh.ksplit == 1) {
    int64_t blocks, units;
    int threads, upw;
    gemv_geometry(sh, epi, a, 1, &units, &upw, &blocks, &threads);
    if (epi == EPI_LINEAR) return launch_s1_two_rows<EPI_LINEAR>(sh, a, units, s);
    if (epi == EPI_QKV) return launch_s1_two_rows<EPI_QKV>(sh, a, units, s);
    if (epi == EPI_SWIGLU) return launch_s1_two_rows<EPI_SWIGLU>(sh, a, units, s);
#if QMM_BITS == 4
    if (epi == EPI_ROPE) return launch_s1_two_rows<EPI_ROPE>(sh, a, units, s);
#endif
  }
  const int64_t batch = M;
  int64_t blocks, units;
  int threads, upw;
  gemv_geometry(sh, epi, a, batch, &units, &upw, &blocks, &threads);
  const dim3 grid{unsigned(blocks), unsigned(M), 1u};
  const dim3 block{unsigned(threads), 1u, 1u};
  if (epi == EPI_LINEAR) {
    QMM_GEMV_CASES(EPI_LINEAR, false)
  } else if (epi == EPI_QKV) {
    QMM_GEMV_CASES(EPI_QKV, false)
  } else if (epi == EPI_ROPE) {
#if QMM_BITS == 4
    QMM_GEMV_CASES(EPI_ROPE, false)
#else
    return 2;  // the rotary epilogue is built for 4-bit codes only
#endif
  } else {
    QMM_GEMV_CASES(EPI_SWIGLU, false)
  }
  return finish_launch();
}

int launch_moe_gate_up(const GemvArgs& a, hipStream_t s) {
  GemvShape sh;
  if (!gemv_shape_for_k(a.K, &sh)) return 2;
  const int64_t batch = a.topk;
  int64_t blocks, units;
  int threads, upw;
  gemv_geometry(sh, EPI_SWIGLU, a, batch, &units, &upw, &blocks, &threads);
  const dim3 grid{unsigned(blocks), unsigned(a.topk), 1u};
  const dim3 block{unsigned(threads), 1u, 1u};
  QMM_GEMV_CASES(EPI_SWIGLU, true)
  return finish_launch();
}

int launch_moe_down(const GemvArgs& a, hipStream_t s) {
  GemvShape sh;
  if (!gemv_shape_for_k(a.K, &sh) || sh.ksplit != 1) return 2;
  const int rpi = 64 / sh.lpr;
  const int64_t units = (a.rows + rpi - 1) / rpi;
  const int kw = a.topk < 8 ? a.topk : 8;
  // about QMM_MOE_DOWN_BLOCKS blocks, at most kMaxUnitsPerCombineBlock units each
  int64_t upw = (units + QMM_MOE_DOWN_BLOCKS - 1) / QMM_MOE_DOWN_BLOCKS;
  if (upw > kMaxUnitsPerCombineBlock) upw = kMaxUnitsPerCombineBlock;
  if (upw < 1) upw = 1;
  const dim3 grid{unsigned((units + upw - 1) / upw), unsigned(a.moe_tokens > 0 ? a.moe_tokens : 1), 1u};
  const dim3 block{unsigned(64 * kw), 1u, 1u};
  switch (sh.lpr * 100 + sh.cpl) {
    case 1601: moe_down_kernel<16, 1><<<grid, block, 0, s>>>(a, units, int(upw)); break;
    case 3201: moe_down_kernel<32, 1><<<grid, block, 0, s>>>(a, units, int(upw)); break;
    case 3202: moe_down_kernel<32, 2><<<grid, block, 0, s>>>(a, units, int(upw)); break;
    case 3203: moe_down_kernel<32, 3><<<grid, block, 0, s>>>(a, units, int(upw)); break;
    case 3204: moe_down_kernel<32, 4><<<grid, block, 0, s>>>(a, units, int(upw)); break;
    case 3205: moe_down_kernel<32, 5><<<grid, block, 0, s>>>(a, units, int(upw)); break;
    default: return 2;
  }
  return finish_launch();
}


}  // namespace QMM_BITS_NS
}  // namespace qmm
