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

namespace qmm {

constexpr int kMaxWavesPerBlock = 16;
constexpr int kUPW = 1;  // row units per wave

template <int LPR, int CPL>
__device__ __forceinline__ void load_x_chunks(const uint16_t* __restrict__ x, int64_t C, int ks, int li,
                                              int64_t cidx[CPL], bool cval[CPL], uint32_t xp[CPL][16],
                                              float xs[CPL]) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int64_t c = int64_t(ks) * (LPR * CPL) + li + LPR * i;
    cval[i] = c < C;
    cidx[i] = cval[i] ? c : (C - 1);
    const uint4* src = reinterpret_cast<const uint4*>(x + cidx[i] * 32);
    uint32_t d[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 t = src[v];
      d[4 * v + 0] = cval[i] ? t.x : 0u;
      d[4 * v + 1] = cval[i] ? t.y : 0u;
      d[4 * v + 2] = cval[i] ? t.z : 0u;
      d[4 * v + 3] = cval[i] ? t.w : 0u;
    }
    permute_chunk(d, xp[i]);
    xs[i] = chunk_xsum(xp[i]);
  }
}

// Partial dot product of one row over this lane's chunks (fp32).
template <int CPL>
__device__ __forceinline__ float row_partial(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                             const uint16_t* __restrict__ biases, int64_t row, int64_t words,
                                             int64_t groups, const int64_t cidx[CPL], const bool cval[CPL],
                                             const uint32_t xp[CPL][16], const float xs[CPL], uint32_t magic) {
  u32x4_t w[CPL];
  uint16_t sb[CPL], bb[CPL];
  const uint32_t* rowp = codes + row * words;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(rowp + cidx[i] * 4));
    sb[i] = scales[row * groups + (cidx[i] >> 1)];
    bb[i] = biases[row * groups + (cidx[i] >> 1)];
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint32_t ww[4] = {w[i][0], w[i][1], w[i][2], w[i][3]};
    const float D = chunk_dot128(ww, xp[i], magic);
    const float d = fmaf(-128.0f, xs[i], D);
    const float s = cval[i] ? bf16_bits_to_f32(sb[i]) : 0.f;
    const float b = cval[i] ? bf16_bits_to_f32(bb[i]) : 0.f;
    acc = fmaf(s, d, acc);
    acc = fmaf(b, xs[i], acc);
  }
  return acc;
}

// Row of the weight handled by slot `slot` of unit `unit`, and whether it exists.
template <int LPR, int EPI>
__device__ __forceinline__ int64_t unit_row(int64_t unit, int slot, const GemvArgs& a, bool* valid) {
  constexpr int RPI = 64 / LPR;
  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int P = RPI / 2;
    const int64_t pair = unit * P + (slot % P);
    *valid = pair < a.I;
    const int64_t r = slot < P ? pair : a.I + pair;
    return *valid ? r : 0;
  } else {
    const int64_t r = unit * RPI + slot;
    *valid = r < a.rows;
    return *valid ? r : (a.rows - 1);
  }
}

// Waves per block: KS waves share each row group; G row groups per block.
template <int KS>
__host__ __device__ constexpr int groups_per_block() { return KS >= 4 ? 1 : 4 / KS; }
template <int KS>
__host__ __device__ constexpr int threads_per_block() { return 64 * KS * groups_per_block<KS>(); }

template <int LPR, int CPL, int KS, int EPI, bool MOE>
__global__ void __launch_bounds__(threads_per_block<KS>()) gemv_u4_kernel(GemvArgs a) {
  constexpr int RPI = 64 / LPR;
  constexpr int P = RPI / 2;
  constexpr int ksplit = KS;
  constexpr int G = groups_per_block<KS>();
  __shared__ float red[kMaxWavesPerBlock * kUPW * RPI];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ks = wave % ksplit;
  const int g = wave / ksplit;
  const int slot = lane / LPR;
  const int li = lane % LPR;
  const int64_t C = a.K >> 5;
  const int64_t words = a.K >> 3;
  const int64_t groups = a.K >> 6;

  const uint32_t* codes = a.codes;
  const uint16_t* scales = a.scales;
  const uint16_t* biases = a.biases;
  const uint16_t* x = a.x;
  int64_t out_base;
  if constexpr (MOE) {
    // blockIdx.y is the routed slot k; its expert's rows are read in place from the grid.
    const int k = blockIdx.y;
    const int32_t e = a.expert_ids[k];
    out_base = int64_t(k) * a.I;
    if (e < 0 || e >= a.E) {
      // no expert: this slot's h is zero
      if (ks == 0) {
        for (int u = 0; u < kUPW; ++u) {
          const int64_t unit = (int64_t(blockIdx.x) * G + g) * kUPW + u;
          bool valid;
          const int64_t r = unit_row<LPR, EPI>(unit, slot, a, &valid);
          (void)r;
          if (valid && slot < P && lane == slot_result_lane<LPR>(slot))
            store_out(a.out0, out_base + unit * P + slot, 0.f, a.f32_out);
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

  int64_t cidx[CPL];
  bool cval[CPL];
  uint32_t xp[CPL][16];
  float xs[CPL];
  load_x_chunks<LPR, CPL>(x, C, ks, li, cidx, cval, xp, xs);
  const uint32_t magic = in_vgpr(kMagicPair);

  float tot[kUPW];
  bool rvalid[kUPW];
  int64_t rrow[kUPW];
#pragma unroll
  for (int u = 0; u < kUPW; ++u) {
    const int64_t unit = (int64_t(blockIdx.x) * G + g) * kUPW + u;
    rrow[u] = unit_row<LPR, EPI>(unit, slot, a, &rvalid[u]);
    const float acc = row_partial<CPL>(codes, scales, biases, rrow[u], words, groups, cidx, cval, xp, xs, magic);
    tot[u] = slot_reduce<LPR>(acc);
  }

  if constexpr (ksplit > 1) {
    if (lane == slot_result_lane<LPR>(slot)) {
#pragma unroll
      for (int u = 0; u < kUPW; ++u) red[(wave * kUPW + u) * RPI + slot] = tot[u];
    }
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int u = 0; u < kUPW; ++u) {
      float v = 0.f;
      for (int j = 0; j < ksplit; ++j) v += red[((g * ksplit + j) * kUPW + u) * RPI + slot];
      tot[u] = v;
    }
  }

#pragma unroll
  for (int u = 0; u < kUPW; ++u) {
    const int64_t unit = (int64_t(blockIdx.x) * G + g) * kUPW + u;
    float v = tot[u];
    if constexpr (EPI == EPI_SWIGLU) {
      const float up = __shfl_xor(v, 32);
      if (rvalid[u] && slot < P && lane == slot_result_lane<LPR>(slot))
        store_out(a.out0, out_base + unit * P + slot, silu_times(v, up), a.f32_out);
    } else {
      if (rvalid[u] && lane == slot_result_lane<LPR>(slot)) {
        const int64_t r = rrow[u];
        if (a.lin_bias) v += bf16_bits_to_f32(a.lin_bias[r]);
        if constexpr (EPI == EPI_QKV) {
          if (r < a.q_out) {
            store_out(a.out0, int64_t(blockIdx.y) * a.q_out + r, v, a.f32_out);
          } else if (r < a.q_out + a.kv_out) {
            store_out(a.out1, int64_t(blockIdx.y) * a.kv_out + (r - a.q_out), v, a.f32_out);
          } else {
            store_out(a.out2, int64_t(blockIdx.y) * a.kv_out + (r - a.q_out - a.kv_out), v, a.f32_out);
          }
        } else {
          store_out(a.out0, out_base + r, v, a.f32_out);
        }
      }
    }
  }
}

// Routed-expert stage 2: y[r] = sum_k p_k * (D_{e_k} h_k)[r].  A block's kw waves split
// the routed slots (wave w takes k = w, w+kw, ...), each adding its slots in increasing
// k; the waves' partials are then added in wave order.  No atomics.
template <int LPR, int CPL>
__global__ void __launch_bounds__(512) moe_down_kernel(GemvArgs a) {
  constexpr int RPI = 64 / LPR;
  __shared__ float red[kMaxWavesPerBlock * kUPW * RPI];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kw = blockDim.x >> 6;
  const int slot = lane / LPR;
  const int li = lane % LPR;
  const int64_t C = a.K >> 5;
  const int64_t words = a.K >> 3;
  const int64_t groups = a.K >> 6;
  const uint32_t magic = in_vgpr(kMagicPair);

  float acc_u[kUPW];
  bool rvalid[kUPW];
  int64_t rrow[kUPW];
#pragma unroll
  for (int u = 0; u < kUPW; ++u) {
    acc_u[u] = 0.f;
    const int64_t r = (int64_t(blockIdx.x) * kUPW + u) * RPI + slot;
    rvalid[u] = r < a.rows;
    rrow[u] = rvalid[u] ? r : a.rows - 1;
  }
  for (int k = wave; k < a.topk; k += kw) {
    const int32_t e = a.expert_ids[k];
    if (e < 0 || e >= a.E) continue;  // no expert: contributes nothing
    const float p = a.expert_w[k];
    int64_t cidx[CPL];
    bool cval[CPL];
    uint32_t xp[CPL][16];
    float xs[CPL];
    load_x_chunks<LPR, CPL>(a.x + int64_t(k) * a.K, C, 0, li, cidx, cval, xp, xs);
    const int64_t off = int64_t(e) * a.rows;
#pragma unroll
    for (int u = 0; u < kUPW; ++u) {
      const float part = row_partial<CPL>(a.codes + off * words, a.scales + off * groups, a.biases + off * groups,
                                          rrow[u], words, groups, cidx, cval, xp, xs, magic);
      acc_u[u] = fmaf(p, slot_reduce<LPR>(part), acc_u[u]);
    }
  }
  if (lane == slot_result_lane<LPR>(slot)) {
#pragma unroll
    for (int u = 0; u < kUPW; ++u) red[(wave * kUPW + u) * RPI + slot] = acc_u[u];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int u = 0; u < kUPW; ++u) {
    if (rvalid[u] && lane == slot_result_lane<LPR>(slot)) {
      float v = 0.f;
      for (int j = 0; j < kw; ++j) v += red[(j * kUPW + u) * RPI + slot];
      store_out(a.out0, rrow[u], v, a.f32_out);
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
  if (cpl > (ks == 16 ? 4 : 5)) return false;
  *o = GemvShape{32, int(cpl), ks};
  return true;
}

static int finish_launch() { return hipGetLastError() == hipSuccess ? 0 : 6; }

#define QMM_GEMV_CASE(L, C, K, EPI, MOE) \
  case (L * 10000 + C * 100 + K): gemv_u4_kernel<L, C, K, EPI, MOE><<<grid, block, 0, s>>>(a); break;

#define QMM_GEMV_CASES(EPI, MOE)                                                  \
  switch (sh.lpr * 10000 + sh.cpl * 100 + sh.ksplit) {                            \
    QMM_GEMV_CASE(16, 1, 1, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 1, 1, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 2, 1, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 3, 1, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 4, 1, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 5, 1, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 1, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 2, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 3, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 4, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 5, 8, EPI, MOE)                                             \
    QMM_GEMV_CASE(32, 3, 16, EPI, MOE)                                            \
    QMM_GEMV_CASE(32, 4, 16, EPI, MOE)                                            \
    default: return 2;                                                            \
  }

static void gemv_geometry(const GemvShape& sh, int epi, const GemvArgs& a, int64_t* blocks, int* threads) {
  const int rpi = 64 / sh.lpr;
  const int64_t units = (epi == EPI_SWIGLU) ? (a.I + rpi / 2 - 1) / (rpi / 2) : (a.rows + rpi - 1) / rpi;
  const int G = sh.ksplit >= 4 ? 1 : 4 / sh.ksplit;  // groups_per_block<KS>()
  *threads = 64 * sh.ksplit * G;
  *blocks = (units + int64_t(G) * kUPW - 1) / (int64_t(G) * kUPW);
}

int launch_gemv(int epi, const GemvArgs& a, int64_t M, hipStream_t s) {
  GemvShape sh;
  if (!gemv_shape_for_k(a.K, &sh)) return 2;
  int64_t blocks;
  int threads;
  gemv_geometry(sh, epi, a, &blocks, &threads);
  const dim3 grid{unsigned(blocks), unsigned(M), 1u};
  const dim3 block{unsigned(threads), 1u, 1u};
  if (epi == EPI_LINEAR) {
    QMM_GEMV_CASES(EPI_LINEAR, false)
  } else if (epi == EPI_QKV) {
    QMM_GEMV_CASES(EPI_QKV, false)
  } else {
    QMM_GEMV_CASES(EPI_SWIGLU, false)
  }
  return finish_launch();
}

int launch_moe_gate_up(const GemvArgs& a, hipStream_t s) {
  GemvShape sh;
  if (!gemv_shape_for_k(a.K, &sh)) return 2;
  int64_t blocks;
  int threads;
  gemv_geometry(sh, EPI_SWIGLU, a, &blocks, &threads);
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
  const dim3 grid{unsigned((units + kUPW - 1) / kUPW), 1u, 1u};
  const dim3 block{unsigned(64 * kw), 1u, 1u};
  switch (sh.lpr * 100 + sh.cpl) {
    case 1601: moe_down_kernel<16, 1><<<grid, block, 0, s>>>(a); break;
    case 3201: moe_down_kernel<32, 1><<<grid, block, 0, s>>>(a); break;
    case 3202: moe_down_kernel<32, 2><<<grid, block, 0, s>>>(a); break;
    case 3203: moe_down_kernel<32, 3><<<grid, block, 0, s>>>(a); break;
    case 3204: moe_down_kernel<32, 4><<<grid, block, 0, s>>>(a); break;
    case 3205: moe_down_kernel<32, 5><<<grid, block, 0, s>>>(a); break;
    default: return 2;
  }
  return finish_launch();
}

}  // namespace qmm
