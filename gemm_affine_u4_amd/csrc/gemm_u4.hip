// Prefill (M > 1) kernel for the u4 group-64 affine quantized projections on gfx950:
// an LDS-dequant + MFMA GEMM.  Prefill is dominated by the quantized matmuls
// ("Sanctum-MLX", latency testing), a dense contraction, so this is the one place the
// path feeds the matrix cores; the fused QKV split and the SwiGLU epilogue follow
// "The Cathedral Doubled Itself" (the two fusions).
//
// Tile: 256 (rows of x) x 256 (rows of the weight) per block of 4 waves, one K step
// = one 64-wide group.  Per step every thread owns one row of each operand tile:
//   * x row: 64 bf16 (128 B) copied to LDS;
//   * weight row: 8 code words + the group's scale and bias; each code becomes
//     w = s*q + b in fp32 (one FMA, exact product), rounded to bf16 (RNE) into LDS.
// Each wave then computes a 128 x 128 sub-tile with v_mfma_f32_32x32x16_bf16 (4 x 4
// tiles of 32 x 32, fp32 accumulators), reading both operands from LDS rows padded to
// 144 B so the 32 rows an MFMA operand spans fall in distinct bank groups.  Two LDS
// buffers: the global loads of step k+1 are in flight while step k is multiplied.
// For SwiGLU a block's 256 weight rows are 128 gate rows and the 128 matching up rows,
// and each wave's columns are 64 gate + the same 64 up columns, so silu(g)*u is formed
// in registers.  Blocks are ordered so the tiles on one XCD (blocks are dealt to the 8
// XCDs round-robin) walk all row tiles of a few weight tiles: the weight tile stays in
// that XCD's L2 while the activation tiles stream.
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;        // rows of x per block
constexpr int kBN = 256;        // weight rows per block
constexpr int kLdsRow = 72;     // bf16 per LDS row (64 + 8 padding)
constexpr int kXcds = 8;

// Byte n of v as a float (v_cvt_f32_ubyte{n}).
template <int n>
__device__ __forceinline__ float ubyte_f32(uint32_t v) { return float((v >> (8 * n)) & 0xFFu); }

// Weight row handled by tile row t (0..255) of weight tile nt.  A row past the end
// maps to the last real row (gate/up pair): its products land in columns that are
// never stored, and every read stays inside the caller's buffers.
template <int EPI>
__device__ __forceinline__ int64_t gemm_weight_row(const GemmArgs& a, int64_t nt, int t) {
  if constexpr (EPI == EPI_SWIGLU) {
    int64_t p = nt * (kBN / 2) + (t & 127);
    if (p >= a.I) p = a.I - 1;
    return t < 128 ? p : a.I + p;
  } else {
    const int64_t n = nt * kBN + t;
    return n < a.N ? n : a.N - 1;
  }
}

template <int EPI>
__global__ void __launch_bounds__(256, 1) gemm_u4_kernel(GemmArgs a, int64_t m_tiles, int64_t n_tiles,
                                                        int64_t tiles_per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLdsRow];

  // XCD-aware tile order: the blocks dealt to XCD x take tiles x*tiles_per_xcd + j,
  // row tiles fastest.
  const int64_t bid = blockIdx.x;
  const int64_t tile = (bid % kXcds) * tiles_per_xcd + bid / kXcds;
  if (tile >= m_tiles * n_tiles) return;
  const int64_t mt = tile % m_tiles;
  const int64_t nt = tile / m_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t K = uint32_t(a.K);
  const uint32_t groups = K >> 6;
  const int ksteps = int(groups);

  // ---- per-thread global sources ----------------------------------------------------
  // x tile of a step: 256 rows x 128 B, read as 2048 16-byte pieces; piece e = 256 j + tid
  // is row e / 8, bytes 16 (e % 8), so eight consecutive threads read one 128-B row.
  // A row past M maps to row M - 1 (never stored).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint64_t(a.M) * K * 2);
  uint32_t xoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int64_t r = mt * kBM + 32 * j + (tid >> 3);
    if (r >= a.M) r = a.M - 1;
    xoff[j] = uint32_t(r) * K * 2 + uint32_t(tid & 7) * 16u;
  }
  // weight tile of a step: thread tid owns weight row tid (8 code words, scale, bias)
  const int64_t wrow = gemm_weight_row<EPI>(a, nt, tid);
  const uint64_t nrows = uint64_t(a.N);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.codes, nrows * (K >> 1));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales, nrows * groups * 2);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.biases, nrows * groups * 2);
  const uint32_t coff = uint32_t(wrow) * (K >> 1);
  const uint32_t goff = uint32_t(wrow) * groups * 2;

  // Global data of one K step, in flight in registers: the x piece of this thread, its
  // weight row's 8 code words and the group's scale and bias.  Two sets alternate, so
  // the loads of step k+2 are issued while step k+1 is dequantized and step k multiplied.
  struct StepRegs {
    u32x4_t xv[8];
    u32x4_t cv[2];
    uint16_t sv, bv;
  };
  StepRegs R[2];
  auto load_step = [&](StepRegs& r, int ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) r.xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[j] + uint32_t(ks) * 128u, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      r.cv[j] = __builtin_amdgcn_raw_buffer_load_b128(cr, coff + uint32_t(ks) * 32u + 16u * j, 0, kLoadNT);
    r.sv = __builtin_amdgcn_raw_buffer_load_b16(sr, goff + uint32_t(ks) * 2u, 0, 0);
    r.bv = __builtin_amdgcn_raw_buffer_load_b16(br, goff + uint32_t(ks) * 2u, 0, 0);
  };
  // Piece p (0..3) of a step into LDS buffer `buf`: x pieces 2p, 2p+1 and code words
  // 2p, 2p+1 (16 codes -> w = s*q + b in fp32 -> bf16, 32 bytes).
  auto store_piece = [&](const StepRegs& r, int buf, int p) {
#pragma unroll
    for (int j = 2 * p; j < 2 * p + 2; ++j)
      *reinterpret_cast<u32x4_t*>(&As[buf][(32 * j + (tid >> 3)) * kLdsRow + (tid & 7) * 8]) = r.xv[j];
    const float s = bf16_bits_to_f32(r.sv);
    const float b = bf16_bits_to_f32(r.bv);
    uint32_t out[8];
#pragma unroll
    for (int ww = 0; ww < 2; ++ww) {
      const uint32_t w = r.cv[p >> 1][2 * (p & 1) + ww];
      // low and high nibbles of the four bytes, then one v_cvt_f32_ubyte{0..3} per code
      const uint32_t lo = in_vgpr(w & 0x0F0F0F0Fu);
      const uint32_t hi = in_vgpr((w >> 4) & 0x0F0F0F0Fu);
      float f[8];
      f[0] = fmaf(s, ubyte_f32<0>(lo), b);
      f[1] = fmaf(s, ubyte_f32<0>(hi), b);
      f[2] = fmaf(s, ubyte_f32<1>(lo), b);
      f[3] = fmaf(s, ubyte_f32<1>(hi), b);
      f[4] = fmaf(s, ubyte_f32<2>(lo), b);
      f[5] = fmaf(s, ubyte_f32<2>(hi), b);
      f[6] = fmaf(s, ubyte_f32<3>(lo), b);
      f[7] = fmaf(s, ubyte_f32<3>(hi), b);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * ww + e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
    }
    u32x4_t* wd = reinterpret_cast<u32x4_t*>(&Bs[buf][tid * kLdsRow]);
    wd[2 * p] = u32x4_t{out[0], out[1], out[2], out[3]};
    wd[2 * p + 1] = u32x4_t{out[4], out[5], out[6], out[7]};
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  // LDS row of the B operand for column tile j of this wave
  auto btile_row = [&](int j) -> int {
    if constexpr (EPI == EPI_SWIGLU) return (j < 2 ? 0 : 128) + 64 * wn + 32 * (j & 1);
    else return 128 * wn + 32 * j;
  };
  const int lr = lane & 31;        // operand row within a 32-row tile
  const int lk = (lane >> 5) * 8;  // first k of this lane's 8 within a 16-wide k step
  struct Frags {
    bf16x8_t a[4], b[4];
  };
  auto load_frags = [&](Frags& f, int buf, int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][(128 * wm + 32 * i + lr) * kLdsRow + kk + lk]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.b[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][(btile_row(j) + lr) * kLdsRow + kk + lk]);
  };
  auto mfma16 = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // One K step: request step ks+2 into register set ks&1, multiply LDS buffer ks&1 (four
  // 16-wide sub-steps, operand fragments of sub-step kk+1 read while kk is multiplied),
  // and between the sub-steps dequantize step ks+1 from set NX = (ks+1)&1 into the
  // other LDS buffer.
  auto kstep = [&](int ks, auto nx_c) {
    constexpr int NX = decltype(nx_c)::value;
    const int buf = ks & 1;
    const bool has_next = ks + 1 < ksteps;
    // step ks was dequantized during the previous step, so its register set is free: request
    // step ks+2 into it now, a whole step ahead of its use
    if (ks + 2 < ksteps) load_step(R[NX ^ 1], ks + 2);
    Frags f[2];
    load_frags(f[0], buf, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q + 1 < 4) load_frags(f[(q + 1) & 1], buf, 16 * (q + 1));
      mfma16(f[q & 1]);
      if (has_next) store_piece(R[NX], buf ^ 1, q);
    }
    __syncthreads();
  };

  load_step(R[0], 0);
  if (ksteps > 1) load_step(R[1], 1);
#pragma unroll
  for (int q = 0; q < 4; ++q) store_piece(R[0], 0, q);
  __syncthreads();
  // step j lives in register set j&1: even steps dequantize set 1, odd steps set 0
  int ks = 0;
  for (; ks + 1 < ksteps; ks += 2) {
    kstep(ks, std::integral_constant<int, 1>{});
    kstep(ks + 1, std::integral_constant<int, 0>{});
  }
  if (ks < ksteps) kstep(ks, std::integral_constant<int, 1>{});

  // ---- epilogue -------------------------------------------------------------------
  // acc[i][j] register r of lane l: row 32i + 8(r/4) + 4(l/32) + r%4 of the wave's rows,
  // column 32j + l%32 of its columns.
  const int64_t row_base = mt * kBM + 128 * wm;
  const int col = lane & 31;
  const int rsub = 4 * (lane >> 5);
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t p = nt * (kBN / 2) + 64 * wn + 32 * j + col;
      if (p >= a.I) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = row_base + 32 * i + 8 * (r >> 2) + rsub + (r & 3);
          if (m < a.M) store_out(a.out0, m * a.I + p, silu_times(acc[i][j][r], acc[i][j + 2][r]), a.f32_out);
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = nt * kBN + 128 * wn + 32 * j + col;
      if (n >= a.N) continue;
      const float lb = a.lin_bias ? bf16_bits_to_f32(a.lin_bias[n]) : 0.f;
      void* dst;
      int64_t cn, ld;
      if constexpr (EPI == EPI_QKV) {
        if (n < a.q_out) {
          dst = a.out0; cn = n; ld = a.q_out;
        } else if (n < a.q_out + a.kv_out) {
          dst = a.out1; cn = n - a.q_out; ld = a.kv_out;
        } else {
          dst = a.out2; cn = n - a.q_out - a.kv_out; ld = a.kv_out;
        }
      } else {
        dst = a.out0; cn = n; ld = a.N;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = row_base + 32 * i + 8 * (r >> 2) + rsub + (r & 3);
          if (m < a.M) store_out(dst, m * ld + cn, acc[i][j][r] + lb, a.f32_out);
        }
    }
  }
}

int launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  const int64_t m_tiles = (a.M + kBM - 1) / kBM;
  const int64_t n_tiles = epi == EPI_SWIGLU ? (a.I + kBN / 2 - 1) / (kBN / 2) : (a.N + kBN - 1) / kBN;
  const int64_t tiles = m_tiles * n_tiles;
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
  const dim3 grid{unsigned(per_xcd * kXcds), 1u, 1u};
  const dim3 block{256u, 1u, 1u};
  if (epi == EPI_LINEAR) {
    gemm_u4_kernel<EPI_LINEAR><<<grid, block, 0, s>>>(a, m_tiles, n_tiles, per_xcd);
  } else if (epi == EPI_QKV) {
    gemm_u4_kernel<EPI_QKV><<<grid, block, 0, s>>>(a, m_tiles, n_tiles, per_xcd);
  } else {
    gemm_u4_kernel<EPI_SWIGLU><<<grid, block, 0, s>>>(a, m_tiles, n_tiles, per_xcd);
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace qmm
