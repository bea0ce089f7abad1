// Prefill (M > 1) kernel for the u4 group-64 affine quantized projections on gfx950:
// an LDS-dequant + MFMA GEMM.  Prefill is dominated by the quantized matmuls
// ("Sanctum-MLX", latency testing), a dense contraction, so this is the one place the
// path feeds the matrix cores; the fused QKV split and the SwiGLU epilogue follow
// "The Cathedral Doubled Itself" (the two fusions).
//
// Tile: 256 (rows of x) x 256 (rows of the weight) per block of 8 waves (two per SIMD), one
// K step = one 64-wide group.  Per step:
//   * x tile (256 rows x 128 B) goes global -> LDS directly (buffer_load ... lds), two
//     steps ahead, into a ring of three LDS stages;
//   * weight tile: each lane owns half of one weight row (4 code words + the group's scale
//     and bias, in registers, requested three steps ahead); each code becomes w = s*q + b
//     in fp32 (one FMA, exact product), rounded to bf16 (RNE) into one of two LDS stages,
//     one step ahead, between the multiplies of the current step.
// Each wave computes a 128 x 64 sub-tile with v_mfma_f32_32x32x16_bf16 (4 x 2 tiles of
// 32 x 32, fp32 accumulators); with two waves per SIMD one wave's MFMAs run while the
// other dequantizes, loads or waits.  LDS rows are 128 B, unpadded; slot c' (16 B) of row
// r holds the row's chunk c' ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1), so the rows an
// MFMA operand read spans (16 consecutive rows at one chunk) hit distinct bank groups.
// Five 32 KB stages fill the 160 KB of LDS.
// For SwiGLU a block's 256 weight rows are 128 gate rows and the 128 matching up rows,
// and each wave's columns are 32 gate + the same 32 up columns, so silu(g)*u is formed
// in registers.  Blocks are ordered so the tiles on one XCD (blocks are dealt to the 8
// XCDs round-robin) walk all row tiles of a few weight tiles: the weight tile stays in
// that XCD's L2 while the activation tiles stream.
#include <type_traits>
#include <utility>

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
constexpr bool kFp8 = QMM_FP8;   // the 8-bit codes are fp8 e4m3 numbers
// vector-memory loads of one lane's 32 codes of a K step (16-, 12- or 8-byte loads)
constexpr int kCodeLoads = kBits / 4 + (kBits % 4 != 0 ? 1 : 0);

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;                 // rows of x per tile
constexpr int kBN = 256;                 // weight rows per tile
constexpr int kRow = 64;                 // bf16 per LDS row (one 64-wide group)
constexpr int kStage = kBN * kRow;       // bf16 per weight stage (32 KB)
constexpr int kXcds = 8;
#ifndef QMM_GEMM_SPLIT_TAIL
#define QMM_GEMM_SPLIT_TAIL 1
#endif
constexpr bool kSplitTail = QMM_GEMM_SPLIT_TAIL;  // the last partial round as half-height blocks

// Bank-group swizzle of LDS row r (see the header).
__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r & 7u) ^ ((r >> 3) & 1u); }

// Byte n of v as a float (v_cvt_f32_ubyte{n}).
template <int n>
__device__ __forceinline__ float ubyte_f32(uint32_t v) { return float((v >> (8 * n)) & 0xFFu); }

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): loop bodies that
// index the accumulator registers with compile-time indices however large they are.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait until at most N of this wave's vector-memory loads are outstanding and its LDS
// operations are done, then meet the other waves.  Written as one asm block (a compiler
// memory barrier) because the compiler's own barrier waits for every outstanding load,
// including the x tile requested for two steps later.
// 16 bytes per lane from buffer r (offset voff + soff) straight into LDS at dst (one wave
// instruction).  A plain function: with the builtin written in the kernel template itself,
// where its arguments depend on the template parameters, the host pass dropped the kernel's
// specializations and left their launch stubs undefined.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint16_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Weight row handled by tile row t (0..255) of weight tile nt.  A row past the end
// maps to the last real row (gate/up pair): its products land in columns that are
// never stored, and every read stays inside the caller's buffers.
template <int EPI>
__device__ __forceinline__ int64_t gemm_weight_row(const GemmArgs& a, int64_t nt, int t) {
  if constexpr (EPI == EPI_SWIGLU) {
    int64_t p = nt * (kBN / 2) + (t & 127);
    if (p >= a.I) p = a.I - 1;
    return t < 128 ? p : a.I + p;
  } else if constexpr (EPI == EPI_ROPE) {
    // rotary QKV: tile rows t and t + 128 are the two rows of pair nt*128 + t
    int64_t p = nt * (kBN / 2) + (t & 127);
    if (p >= (a.N >> 1)) p = (a.N >> 1) - 1;
    const RopePair rp = rope_pair(uint32_t(p), a.rope);
    return t < 128 ? rp.ra : rp.rb;
  } else {
    const int64_t n = nt * kBN + t;
    return n < a.N ? n : a.N - 1;
  }
}

// BM = kBM: a block computes a whole 256 x 256 tile.  BM = kBM / 2: a block computes half
// of one (128 rows of x, rows 128 h .. of the tile for half h) against the whole weight tile,
// which it dequantizes in full: used for a last round of tiles that would leave more than
// half of the CUs idle, so that it runs in about the time of the half-height blocks.
template <int EPI, int BM>
__global__ void __launch_bounds__(512, 1) gemm_u4_kernel(GemmArgs a, int64_t m_tiles, int64_t tile0,
                                                        int64_t units, int64_t units_per_xcd) {
  constexpr int kSplit = kBM / BM;      // blocks per tile
  constexpr int kI = BM / 64;           // 32-row x sub-tiles per wave (4 or 2)
  constexpr int kXStage = BM * kRow;    // bf16 per x stage
  // One variable per x stage, and the two weight stages in a variable of their own: the
  // compiler then knows that the x stage being filled by a direct-to-LDS load aliases
  // neither the x stage nor the weight stage being read.
  __shared__ __attribute__((aligned(1024))) uint16_t As0[kXStage], As1[kXStage], As2[kXStage];
  __shared__ __attribute__((aligned(1024))) uint16_t Bs[2 * kStage];

  // XCD-aware order: the blocks dealt to XCD x take units x*units_per_xcd + j (a unit is a
  // tile, or half of one; the halves of a tile are consecutive, so they share the XCD and its
  // L2 copy of the weight tile), tiles from tile0 on, row tiles fastest.
  const int64_t bid = blockIdx.x;
  const int64_t unit = (bid % kXcds) * units_per_xcd + bid / kXcds;
  if (unit >= units) return;
  const int64_t tile = tile0 + unit / kSplit;
  const int64_t mt = tile % m_tiles;
  const int64_t nt = tile / m_tiles;
  const int64_t xrow0 = mt * kBM + (unit % kSplit) * BM;  // first x row of the block

  // source row of block row r (x rows [xrow0, xrow0 + BM); a row past M reads row M - 1,
  // never stored)
  auto x_row = [&](int r) -> int64_t {
    const int64_t m = xrow0 + r;
    return m < a.M ? m : a.M - 1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const uint32_t K = uint32_t(a.K);
  const int ksteps = int(K >> 6);
  const uint32_t groups = K >> (5 + a.gshift);  // scale/bias groups per row (group 32 << gshift)

  // ---- x tile: global -> LDS ----------------------------------------------------------
  // Instruction j (j < kI) of wave w fills LDS rows (BM / 8) w + 8 j + L / 8, slot L % 8 (lane
  // L lands at byte 16 L); that slot holds chunk (L % 8) ^ swz(row) = (L % 8) ^ (L / 8) ^ (j & 1).
  // A row past M reads row M - 1 (never stored).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint64_t(a.M) * K * 2);
  uint32_t xoff[kI];
#pragma unroll
  for (int j = 0; j < kI; ++j) {
    const int64_t r = x_row((BM / 8) * wave + 8 * j + (lane >> 3));
    const uint32_t chunk = uint32_t((lane & 7) ^ (lane >> 3) ^ (j & 1));
    xoff[j] = uint32_t(r) * K * 2 + chunk * 16u;
  }
  auto x_stage = [&](auto p_c) -> uint16_t* {
    constexpr int P = decltype(p_c)::value;
    return P == 0 ? As0 : (P == 1 ? As1 : As2);
  };
  auto load_x = [&](uint16_t* dst, int ks) {
#pragma unroll
    for (int j = 0; j < kI; ++j) load_lds16(xr, dst + ((BM / 8) * wave + 8 * j) * kRow, xoff[j], uint32_t(ks) * 128u);
  };

  // ---- weight tile: global -> registers -> dequant -> LDS -----------------------------
  // Two lanes per weight row: in load i (0, 1) lane L reads half L / 32 (16 B, 32 codes) of
  // the step's codes of tile row 64 w + 32 i + L % 32, so one wave load touches 32 rows.
  // The lane then dequantizes those 32 codes into chunks 4 (L / 32) .. +3 of that row.
  const int wh = lane >> 5;
  const uint64_t nrows = uint64_t(a.N);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.codes, nrows * ((K * kBits) >> 3));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales, nrows * groups * 2);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.biases, nrows * groups * 2);
  const int wt = 32 * wave + (lane & 31);  // tile row whose half `wh` this lane owns
  const int64_t wrow = gemm_weight_row<EPI>(a, nt, wt);
  // codes of row wrow: K*bits/8 bytes; the lane's 32 codes of step ks start 4*bits bytes
  // into the step's 8*bits
  const uint32_t coff = uint32_t(wrow) * ((K * kBits) >> 3) + uint32_t(4 * kBits) * uint32_t(wh);
  const uint32_t goff = uint32_t(wrow) * groups * 2;
  const uint32_t wdst = uint32_t(wt) * kRow;
  const uint32_t wsw = swz(uint32_t(wt));
  // one step of this lane's half row in flight: its bits code words, scale, bias; step j
  // lives in set j % 3
  struct StepRegs {
    uint32_t cv[kBits];
    uint16_t sv, bv;
  };
  StepRegs R[3];
  // the lane's 32 codes of step ks are inputs 64 ks + 32 wh .. +31: group (2 ks + wh) >> gshift
  auto load_w = [&](StepRegs& r, int ks) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
    const uint32_t go = goff + ((uint32_t(2 * ks + wh) >> a.gshift) << 1);
    const uint32_t co = coff + uint32_t(ks) * uint32_t(8 * kBits);
    int i = 0;
#pragma unroll
    for (; i + 4 <= kBits; i += 4) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(cr, co + 4u * i, 0, 0);
      r.cv[i] = v[0];
      r.cv[i + 1] = v[1];
      r.cv[i + 2] = v[2];
      r.cv[i + 3] = v[3];
    }
    if constexpr (kBits % 4 == 3) {
      const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(cr, co + 4u * i, 0, 0);
      r.cv[i] = v[0];
      r.cv[i + 1] = v[1];
      r.cv[i + 2] = v[2];
    } else if constexpr (kBits % 4 == 2) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(cr, co + 4u * i, 0, 0);
      r.cv[i] = v[0];
      r.cv[i + 1] = v[1];
    }
    r.sv = __builtin_amdgcn_raw_buffer_load_b16(sr, go, 0, 0);
    r.bv = __builtin_amdgcn_raw_buffer_load_b16(br, go, 0, 0);
  };
  constexpr int kStepLoads = kI + kCodeLoads + 2;  // vector-memory loads one step requests per lane
  // Piece p (0..3): codes 8p .. 8p+7 of the half row (-> w = s*q + b in fp32 -> bf16, 16
  // bytes) into chunk 4 wh + p of the row in stage `dst`.
  auto store_piece = [&](const StepRegs& r, uint16_t* dst, int p) {
    const float s = bf16_bits_to_f32(r.sv);
    const float b = bf16_bits_to_f32(r.bv);
    u32x4_t v;
    if constexpr (kFp8) {
      // codes 8p .. 8p+7 are the bytes of words 2p, 2p+1: two e4m3 -> fp32 per conversion
      typedef float f32x2_t __attribute__((ext_vector_type(2)));
      const uint32_t w0 = r.cv[2 * p], w1 = r.cv[2 * p + 1];
      const f32x2_t c0 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false), c1 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
      const f32x2_t c2 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false), c3 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
      v = u32x4_t{pack_bf16x2(fmaf(s, c0[0], b), fmaf(s, c0[1], b)), pack_bf16x2(fmaf(s, c1[0], b), fmaf(s, c1[1], b)),
                  pack_bf16x2(fmaf(s, c2[0], b), fmaf(s, c2[1], b)), pack_bf16x2(fmaf(s, c3[0], b), fmaf(s, c3[1], b))};
    } else if constexpr (kBits == 4) {
      // low and high nibbles of the four bytes of word p, one v_cvt_f32_ubyte{0..3} per code
      const uint32_t w = r.cv[p];
      const uint32_t lo = in_vgpr(w & 0x0F0F0F0Fu);
      const uint32_t hi = in_vgpr((w >> 4) & 0x0F0F0F0Fu);
      v = u32x4_t{pack_bf16x2(fmaf(s, ubyte_f32<0>(lo), b), fmaf(s, ubyte_f32<0>(hi), b)),
                  pack_bf16x2(fmaf(s, ubyte_f32<1>(lo), b), fmaf(s, ubyte_f32<1>(hi), b)),
                  pack_bf16x2(fmaf(s, ubyte_f32<2>(lo), b), fmaf(s, ubyte_f32<2>(hi), b)),
                  pack_bf16x2(fmaf(s, ubyte_f32<3>(lo), b), fmaf(s, ubyte_f32<3>(hi), b))};
    } else if constexpr (kBits == 8) {
      // the bytes of words 2p and 2p + 1 are the codes
      const uint32_t w0 = r.cv[2 * p], w1 = r.cv[2 * p + 1];
      v = u32x4_t{pack_bf16x2(fmaf(s, ubyte_f32<0>(w0), b), fmaf(s, ubyte_f32<1>(w0), b)),
                  pack_bf16x2(fmaf(s, ubyte_f32<2>(w0), b), fmaf(s, ubyte_f32<3>(w0), b)),
                  pack_bf16x2(fmaf(s, ubyte_f32<0>(w1), b), fmaf(s, ubyte_f32<1>(w1), b)),
                  pack_bf16x2(fmaf(s, ubyte_f32<2>(w1), b), fmaf(s, ubyte_f32<3>(w1), b))};
    } else {
      // code k of the half row: stream bits [bits*k, bits*k + bits) (may straddle words)
      constexpr uint32_t m = (1u << kBits) - 1u;
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = fmaf(s, float(stream_window(r.cv, kBits * (8 * p + j)) & m), b);
      v = u32x4_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                  pack_bf16x2(f[6], f[7])};
    }
    const uint32_t chunk = uint32_t(4 * wh + p);
    *reinterpret_cast<u32x4_t*>(dst + wdst + (chunk ^ wsw) * 8) = v;
  };

  // ---- MFMA operands from LDS ---------------------------------------------------------
  f32x16_t acc[kI][2];
#pragma unroll
  for (int i = 0; i < kI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  // LDS row of the B operand for column tile j of this wave
  auto btile_row = [&](int j) -> int {
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_ROPE) return (j == 0 ? 0 : 128) + 32 * wn;
    else return 64 * wn + 32 * j;
  };
  // Operand lane l holds row l % 32 of a 32-row tile and k 8 (l / 32) .. +7 of a 16-wide
  // sub-step q, i.e. chunk 2q + l / 32 of the row; tiles start at multiples of 32 rows,
  // so swz(row) = swz(l % 32) and one offset per q serves every tile of both operands.
  const uint32_t lr = uint32_t(lane & 31);
  uint32_t opoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) opoff[q] = lr * kRow + (uint32_t(2 * q + (lane >> 5)) ^ swz(lr)) * 8u;
  struct Frags {
    bf16x8_t a[kI], b[2];
  };
  auto load_frags = [&](Frags& f, const uint16_t* as, const uint16_t* bs, int q) {
#pragma unroll
    for (int i = 0; i < kI; ++i) f.a[i] = *reinterpret_cast<const bf16x8_t*>(as + ((BM / 2) * wm + 32 * i) * kRow + opoff[q]);
#pragma unroll
    for (int j = 0; j < 2; ++j) f.b[j] = *reinterpret_cast<const bf16x8_t*>(bs + btile_row(j) * kRow + opoff[q]);
  };
  auto mfma16 = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };

  // Instruction order inside a slot: the wave issues in order and an MFMA waits for the
  // matrix pipe, so the dequantization's ~24 VALU ops are spread 3 per MFMA (they then
  // run while the MFMA executes) and its LDS store goes late in the slot.
  auto interleave_slot = [&]() {
    constexpr int kMfma = 2 * kI;  // MFMAs per slot
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 24 / kMfma, 0);    // its share of the VALU
      if (i == kMfma - 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // the LDS store
    }
  };

  // K loop.  Step j's x tile lives in x stage j % 3, its dequantized weights in weight
  // stage j & 1, its raw weights in register set j % 3.  Each step is four slots of 8
  // MFMAs (one 16-wide sub-step each); in every slot the operand fragments of the next
  // sub-step are read from LDS and a quarter of the next step's weights is dequantized.
  // The one barrier of a step, X, sits before its last slot, when every fragment of the
  // step has been read into registers: after X the step's x and weight stages are free,
  // and the first fragments of the next step are read while the last 8 MFMAs run.
  // Before X a wave waits for its x of the next step and the raw weights of the one after,
  // requested after the barrier two steps back: only the loads requested after the
  // previous barrier (kStepLoads) may still be in flight.  Requested steps are clamped to
  // the last one, so every step issues the same loads and nothing branches; the extra
  // copies land in stages and registers that are never read again.
  Frags f[2];
  auto iteration = [&](int ks, auto p_c) {
    constexpr int P = decltype(p_c)::value;
    const uint16_t* as = x_stage(p_c);
    const uint16_t* bs = Bs + (ks & 1) * kStage;
    uint16_t* bnext = Bs + ((ks + 1) & 1) * kStage;
    // slots 0..2: sub-steps 0..2 of step ks, pieces 1..3 of step ks+1's weights
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      load_frags(f[(q + 1) & 1], as, bs, q + 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma16(f[q & 1]);
      store_piece(R[(P + 1) % 3], bnext, q + 1);
      interleave_slot();
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_loads_barrier<kStepLoads>();
    // x stage P and weight stage ks & 1 are free: request x of step ks+3 and the weights
    // of step ks+4 (register set (ks+1) % 3, whose step was just dequantized)
    load_x(x_stage(p_c), min(ks + 3, ksteps - 1));
    load_w(R[(P + 1) % 3], min(ks + 4, ksteps - 1));
    // slot 3: sub-step 3 of step ks, fragments of step ks+1's sub-step 0, piece 0 of step
    // ks+2's weights into the freed weight stage
    load_frags(f[0], x_stage(std::integral_constant<int, (P + 1) % 3>{}), bnext, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(f[1]);
    store_piece(R[(P + 2) % 3], Bs + (ks & 1) * kStage, 0);
    interleave_slot();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue, ending in the state an iteration expects: x of steps 0 and 1 and the raw
  // weights of steps 1 and 2 landed or in flight as if requested two and one barriers
  // back, step 0 dequantized and published, x of step 2 and weights of step 3 requested
  // after the last barrier, step 0's first fragments read and step 1's first piece
  // dequantized.
  load_x(As0, 0);
  load_w(R[0], 0);
  load_w(R[1], min(1, ksteps - 1));
  __builtin_amdgcn_s_waitcnt(0);  // the compiler accounts for this full wait too
#pragma unroll
  for (int p = 0; p < 4; ++p) store_piece(R[0], Bs, p);
  load_x(As1, min(1, ksteps - 1));
  load_w(R[2], min(2, ksteps - 1));
  wait_loads_barrier<kStepLoads>();
  load_x(As2, min(2, ksteps - 1));
  load_w(R[0], min(3, ksteps - 1));
  load_frags(f[0], As0, Bs, 0);
  store_piece(R[1], Bs + kStage, 0);
  int ks = 0;
  for (; ks + 2 < ksteps; ks += 3) {
    iteration(ks, std::integral_constant<int, 0>{});
    iteration(ks + 1, std::integral_constant<int, 1>{});
    iteration(ks + 2, std::integral_constant<int, 2>{});
  }
  if (ks < ksteps) iteration(ks, std::integral_constant<int, 0>{});
  if (ks + 1 < ksteps) iteration(ks + 1, std::integral_constant<int, 1>{});

  // ---- epilogue -------------------------------------------------------------------
  // The MFMA takes the weight fragment as its first operand, so acc[i][j] is the
  // transposed tile: register r of lane l holds output row 32i + l%32 of the wave's rows
  // and output column (weight row) 32j + 8(r/4) + 4(l/32) + r%4 of the wave's columns.
  // A lane thus owns 4 consecutive columns of one row per register quad and writes them
  // with one 8-byte (bf16) or 16-byte (fp32) store where they share a destination and the
  // address is aligned, element by element otherwise (ragged edges, odd row strides).
  const int trow0 = (BM / 2) * wm + (lane & 31);  // block row of this lane's output row, i = 0
  const int csub = 4 * (lane >> 5);
  // output row of tile row trow0 + 32 i, false if the row does not exist
  auto out_row = [&](int i, int64_t* m) -> bool {
    *m = xrow0 + trow0 + 32 * i;
    return *m < a.M;
  };
  // 4 consecutive outputs from element idx: one vector store when all 4 exist and the
  // address is aligned to it (the ABI only promises element alignment of the buffer)
  auto put = [&](void* dst, int64_t ld, int64_t cn, int64_t m, const float (&v)[4], int nvalid) {
    const int64_t idx = m * ld + cn;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(dst) + uintptr_t(idx) * (a.f32_out ? 4u : 2u);
    if (nvalid == 4 && (addr & (a.f32_out ? 15u : 7u)) == 0) {
      if (a.f32_out) {
        *reinterpret_cast<float4*>(static_cast<float*>(dst) + idx) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + idx) =
            make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                       f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < nvalid) store_out(dst, idx + e, v[e], a.f32_out);
    }
  };
  if constexpr (EPI == EPI_ROPE) {
    // Pair p's two rows are columns p0 + e of acc[i][0] and acc[i][1]; each is rotated (or
    // passed through) and stored into its head of q/k/v/gate.  When head_dim and rot are
    // multiples of 8, the 4 pairs p0 .. p0+3 of a lane (p0 % 4 == 0) lie in one head and
    // one region (rotated or not), so their dims are consecutive: one 16-byte read of
    // cos and of sin, and 4-element stores.
    const RopeArgs& ra = a.rope;
    const bool grouped = (ra.head_dim % 8) == 0 && (ra.rot % 8) == 0;
    int64_t mrow[4];
    const float* trow[4];
    bool have[4];
#pragma unroll
    for (int i = 0; i < kI; ++i) {
      have[i] = out_row(i, &mrow[i]);
      const int32_t pos = have[i] ? min(max(ra.positions[mrow[i]], 0), ra.max_pos - 1) : 0;
      trow[i] = ra.cos_sin + int64_t(pos) * ra.rot;
    }
    static_for<4>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      const int64_t p0 = nt * (kBN / 2) + 32 * wn + 8 * g + csub;
      if (p0 >= (a.N >> 1)) return;
      if (grouped) {
        const RopePair rp = rope_pair(uint32_t(p0), ra);
        float lba[4], lbb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lba[e] = a.lin_bias ? bf16_bits_to_f32(a.lin_bias[rp.ra + e]) : 0.f;
          lbb[e] = a.lin_bias ? bf16_bits_to_f32(a.lin_bias[rp.rb + e]) : 0.f;
        }
        void* dst;
        int64_t nh;
        switch (rp.buf) {
          case ROPE_Q: dst = a.out0; nh = ra.n_q; break;
          case ROPE_K: dst = a.out1; nh = ra.n_kv; break;
          case ROPE_V: dst = a.out2; nh = ra.n_kv; break;
          default: dst = ra.gate; nh = ra.n_q; break;
        }
#pragma unroll
        for (int i = 0; i < kI; ++i) {
          if (!have[i]) continue;
          float va[4], vb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            va[e] = acc[i][0][4 * g + e] + lba[e];
            vb[e] = acc[i][1][4 * g + e] + lbb[e];
          }
          if (rp.ri >= 0) {
            const float4 c = *reinterpret_cast<const float4*>(trow[i] + rp.ri);
            const float4 sn = *reinterpret_cast<const float4*>(trow[i] + (ra.rot >> 1) + rp.ri);
            const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x0 = va[e], x1 = vb[e];
              va[e] = fmaf(x0, cc[e], -(x1 * ss[e]));
              vb[e] = fmaf(x1, cc[e], x0 * ss[e]);
            }
          }
          const int64_t base = (mrow[i] * nh + rp.head) * int64_t(ra.head_dim);
          put(dst, 0, base + rp.da, 0, va, 4);
          put(dst, 0, base + rp.db, 0, vb, 4);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t p = p0 + e;
          if (p >= (a.N >> 1)) continue;
          const RopePair rp = rope_pair(uint32_t(p), ra);
          const float lba = a.lin_bias ? bf16_bits_to_f32(a.lin_bias[rp.ra]) : 0.f;
          const float lbb = a.lin_bias ? bf16_bits_to_f32(a.lin_bias[rp.rb]) : 0.f;
#pragma unroll
          for (int i = 0; i < kI; ++i) {
            if (!have[i]) continue;
            rope_store(ra, a.out0, a.out1, a.out2, rp, mrow[i], acc[i][0][4 * g + e] + lba,
                       acc[i][1][4 * g + e] + lbb, a.f32_out);
          }
        }
      }
    });
  } else if constexpr (EPI == EPI_SWIGLU) {
    static_for<4>([&](auto gc) {
      constexpr int j = 0, g = decltype(gc)::value;
      {
        const int64_t p0 = nt * (kBN / 2) + 32 * wn + 8 * g + csub;
        if (p0 >= a.I) return;
        const int nvalid = int(min<int64_t>(4, a.I - p0));
#pragma unroll
        for (int i = 0; i < kI; ++i) {
          int64_t m;
          if (!out_row(i, &m)) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = silu_times(acc[i][j][4 * g + e], acc[i][j + 1][4 * g + e]);
          put(a.out0, a.I, p0, m, v, nvalid);
        }
      }
    });
  } else {
    // output column n -> destination, row stride, column there, end of its range
    auto route = [&](int64_t n, void*& dst, int64_t& ld, int64_t& cn, int64_t& end) {
      if constexpr (EPI == EPI_QKV) {
        if (n < a.q_out) {
          dst = a.out0; ld = a.q_out; cn = n; end = a.q_out;
        } else if (n < a.q_out + a.kv_out) {
          dst = a.out1; ld = a.kv_out; cn = n - a.q_out; end = a.q_out + a.kv_out;
        } else {
          dst = a.out2; ld = a.kv_out; cn = n - a.q_out - a.kv_out; end = a.N;
        }
      } else {
        dst = a.out0; ld = a.N; cn = n; end = a.N;
      }
    };
    static_for<8>([&](auto jg) {
      constexpr int j = decltype(jg)::value / 4, g = decltype(jg)::value % 4;
      {
        const int64_t n0 = nt * kBN + 64 * wn + 32 * j + 8 * g + csub;
        if (n0 >= a.N) return;
        float lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lb[e] = (a.lin_bias && n0 + e < a.N) ? bf16_bits_to_f32(a.lin_bias[n0 + e]) : 0.f;
        void* dst;
        int64_t ld, cn, end;
        route(n0, dst, ld, cn, end);
        const bool one_range = n0 + 3 < end;
#pragma unroll
        for (int i = 0; i < kI; ++i) {
          int64_t m;
          if (!out_row(i, &m)) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] + lb[e];
          if (one_range) {
            put(dst, ld, cn, m, v, 4);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (n0 + e >= a.N) continue;
              void* d1;
              int64_t ld1, cn1, end1;
              route(n0 + e, d1, ld1, cn1, end1);
              store_out(d1, m * ld1 + cn1, v[e], a.f32_out);
            }
          }
        }
      }
    });
  }
}

// One launch over tiles [tile0, tile0 + tiles) of the grid, each as one block (half = false)
// or as two half-height blocks.
static int launch_tiles(int epi, bool half, const GemmArgs& a, int64_t m_tiles, int64_t tile0, int64_t tiles,
                        hipStream_t s) {
  const int64_t split = half ? 2 : 1;
  const int64_t units = tiles * split;
  // whole tiles per XCD range, so that the halves of a tile land on one XCD
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds * split;
  const dim3 grid{unsigned(per_xcd * kXcds), 1u, 1u};
  const dim3 block{512u, 1u, 1u};
#define QMM_GEMM_LAUNCH(E)                                                                          \
  do {                                                                                              \
    if (half) gemm_u4_kernel<E, kBM / 2><<<grid, block, 0, s>>>(a, m_tiles, tile0, units, per_xcd); \
    else gemm_u4_kernel<E, kBM><<<grid, block, 0, s>>>(a, m_tiles, tile0, units, per_xcd);          \
  } while (0)
  if (epi == EPI_LINEAR) {
    QMM_GEMM_LAUNCH(EPI_LINEAR);
  } else if (epi == EPI_QKV) {
    QMM_GEMM_LAUNCH(EPI_QKV);
  } else if (epi == EPI_ROPE) {
#if QMM_BITS == 4
    QMM_GEMM_LAUNCH(EPI_ROPE);
#else
    return 2;  // the rotary epilogue is built for 4-bit codes only
#endif
  } else {
    QMM_GEMM_LAUNCH(EPI_SWIGLU);
  }
#undef QMM_GEMM_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// One block per CU: after the whole rounds of tiles, a remainder of at most half the CUs
// runs as half-height blocks (two per tile) in a launch of its own, which fills up to all
// of the CUs and takes about the time of one such block instead of a whole tile.
int launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  const int64_t m_tiles = (a.M + kBM - 1) / kBM;
  const int64_t n_tiles = epi == EPI_SWIGLU ? (a.I + kBN / 2 - 1) / (kBN / 2)
                          : epi == EPI_ROPE ? ((a.N >> 1) + kBN / 2 - 1) / (kBN / 2)
                                            : (a.N + kBN - 1) / kBN;
  const int64_t tiles = m_tiles * n_tiles;
  const int64_t cus = device_cus();
  const int64_t rem = tiles % cus;
  if (kSplitTail && tiles > cus && rem > 0 && 2 * rem <= cus) {
    if (int st = launch_tiles(epi, false, a, m_tiles, 0, tiles - rem, s)) return st;
    return launch_tiles(epi, true, a, m_tiles, tiles - rem, rem, s);
  }
  return launch_tiles(epi, false, a, m_tiles, 0, tiles, s);
}

}  // namespace QMM_BITS_NS
}  // namespace qmm
