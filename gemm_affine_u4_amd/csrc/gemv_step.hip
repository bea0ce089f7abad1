// A decode step in few launches: several 4-bit group-64 projections of one token (fused QKV,
// fused gate+up+SwiGLU, plain projections such as the down projection) run by one launch per
// dependency level and kind instead of one launch per projection.  The pages fuse projections
// because a decode step is launch-bound as much as bandwidth-bound (96 launches ~ 3 ms per
// step: "The Cathedral Doubled Itself", the two fusions); saragossa submits one command
// buffer per token (saragossa README, design principles).  Here the 14B-shaped step (fused QKV
// + fused gate+up) is one launch, and a 24B-shaped step of 40 layers (120 projections, the
// down projections reading their layer's h) is two.
//
// Grouping and work lists: see qmm_step.h.  Every position is computed with exactly the
// arithmetic of the per-call decode kernels (gemv_u4.hip) for that projection's K: the same
// lanes own the same 32-code chunks, the same fp32 operations in the same order, the same
// lane reduction, and a K split over waves adds the waves' partials in wave order from zero.
// So every output equals the per-call result bit for bit.
//
// Why no launch waits inside itself: ordering two projections inside one launch takes a
// device-scope counter and release/acquire across the XCDs' L2 caches per producing and
// consuming wave; measured on MI355X that costs ~45 ns of serialised work per wave and event
// (an atomic on one address ~12 ns), hundreds of microseconds per 24B-shaped step, against
// ~2 us for a second launch.
#include "qmm.h"
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_step.h"
#include "qmm_validate.h"

#include <algorithm>
#include <vector>

namespace qmm {
namespace step {

constexpr int LPR = 32;     // lanes per row slot (two rows per wave)
constexpr int kMaxCpl = 5;  // 32-code chunks per lane in a slice, at most
constexpr int kXStride = 20;                 // words per staged activation chunk (16 + 4 padding)
constexpr int kMaxChunks = LPR * kMaxCpl;    // chunks of a single-slice K (K <= 5120)
constexpr int kXWords = kMaxChunks * kXStride + kMaxChunks;  // permuted chunks, then chunk sums

// Values the whole wave shares, made visibly uniform (scalar registers): the compiler cannot
// always prove it through the plan's index chain, and a buffer descriptor it takes for
// per-lane makes every load a loop over lanes.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T* uni_ptr(T* p) {
  return reinterpret_cast<T*>(uni64(int64_t(reinterpret_cast<uintptr_t>(p))));
}

template <int CPL>
struct RowBuf {
  uint32_t w[CPL][4];
  uint16_t s[CPL], b[CPL];
};

// The codes, scales and biases of one row for this lane's chunks c0 + 32 i, i < CPL (the
// per-call kernels' load_row at 4 bits, group 64: chunks 512 bytes and groups 32 bytes apart).
template <int CPL>
__device__ __forceinline__ void load_unit(RowBuf<CPL>& r, __amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr,
                                          __amdgpu_buffer_rsrc_t br, uint32_t row, uint32_t row_bytes,
                                          uint32_t row_groups, uint32_t c0) {
  const uint32_t co = row * row_bytes + c0 * 16u;
  const uint32_t go = (row * row_groups + (c0 >> 1)) * 2u;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(cr, co + uint32_t(i) * 512u, 0, kLoadNT);
    r.w[i][0] = v[0];
    r.w[i][1] = v[1];
    r.w[i][2] = v[2];
    r.w[i][3] = v[3];
    r.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, go + uint32_t(i) * 32u, 0, 0);
    r.b[i] = __builtin_amdgcn_raw_buffer_load_b16(br, go + uint32_t(i) * 32u, 0, 0);
  }
}

// Activations of chunks c0 + 32 i (zero past K), permuted to the nibble-pair order, and
// their chunk sums.
template <int CPL>
__device__ __forceinline__ void load_x(uint32_t xp[CPL][16], float xs[CPL], __amdgpu_buffer_rsrc_t xr, uint32_t c0) {
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
    permute_chunk(d, xp[i]);
    xs[i] = chunk_xsum(xp[i]);
    // one chunk's raw activations at a time: keeps the entry of a segment from holding all
    // of them in registers next to the permuted ones
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Partial dot product of one row over this lane's chunks (the per-call row_partial).
template <int CPL>
__device__ __forceinline__ float unit_partial(const RowBuf<CPL>& r, const uint32_t xp[CPL][16], const float xs[CPL],
                                              uint32_t magic) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const float d = fmaf(-128.0f, xs[i], chunk_dot128(r.w[i], xp[i], magic));
    acc = fmaf(bf16_bits_to_f32(r.s[i]), d, acc);
    acc = fmaf(bf16_bits_to_f32(r.b[i]), xs[i], acc);
  }
  return acc;
}

__device__ __forceinline__ void store_qkv(const Proj& P, int64_t r, float v) {
  if (r < P.q_out) {
    store_out(P.out0, r, v, P.f32_out);
  } else if (r < P.q_out + P.kv_out) {
    store_out(P.out1, r - P.q_out, v, P.f32_out);
  } else {
    store_out(P.out2, r - P.q_out - P.kv_out, v, P.f32_out);
  }
}

// Weight row of slot `slot` in unit u, and whether it exists: a (gate, up) pair for SwiGLU,
// two consecutive rows otherwise.
template <bool SWIGLU>
__device__ __forceinline__ uint32_t unit_row(const Proj& P, uint32_t u, int slot, bool* valid) {
  const uint32_t r = SWIGLU ? (slot == 0 ? u : uint32_t(P.I) + u) : u * 2 + slot;
  *valid = SWIGLU ? u < uint32_t(P.I) : r < uint32_t(P.rows);
  return r;
}

// ---- single-slice launches (K <= 5120) ------------------------------------------------------

// Stage the activations of x[0 .. K) in LDS for lanes reading cpl chunks each: chunk c < 32 cpl
// (32 values, zero past K) permuted to the nibble-pair order at xl + c * kXStride, its sum at
// xl + kMaxChunks * kXStride + c.  All threads of the block take part.
__device__ __forceinline__ void stage_x(uint32_t* xl, const uint16_t* x, int K, int cpl) {
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(uni_ptr(x), uint64_t(uni(K)) * 2);
  float* xsl = reinterpret_cast<float*>(xl + kMaxChunks * kXStride);
  const int C = LPR * cpl;  // every chunk a lane reads (zeros past K)
  for (int c = threadIdx.x; c < C; c += 64 * kWavesPerBlockSingle) {
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
    permute_chunk(d, xp);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(xl + c * kXStride);
#pragma unroll
    for (int v = 0; v < 4; ++v) dst[v] = u32x4_t{xp[4 * v], xp[4 * v + 1], xp[4 * v + 2], xp[4 * v + 3]};
    xsl[c] = chunk_xsum(xp);
  }
}

// This wave's chunks (c0 + 32 i) of staged activations into registers.
template <int CPL>
__device__ __forceinline__ void x_from_lds(uint32_t xp[CPL][16], float xs[CPL], const uint32_t* xl, uint32_t c0) {
  const float* xsl = reinterpret_cast<const float*>(xl + kMaxChunks * kXStride);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint32_t c = c0 + uint32_t(LPR * i);
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
}

// This wave's positions p, p + 4, ... below end of one projection (positions = row units,
// the projection's first at seg_begin), with the activations from the block's LDS copy xl
// (LDS_X) or from memory.  `before_x` runs once the first unit's weights are requested and
// before the activations are read (the block's staging, on the wave's first projection).
// Returns the wave's first position at or past end.
template <int CPL, bool SWIGLU, bool LDS_X, typename BeforeX>
__device__ __forceinline__ int64_t run_single(const Proj P, int64_t p, int64_t seg_begin, int64_t end,
                                              const uint32_t* xl, BeforeX&& before_x) {
  const int lane = threadIdx.x & 63;
  const int slot = lane / LPR;
  const int li = lane % LPR;
  const bool result_lane = lane == slot_result_lane<LPR>(slot);
  const uint32_t magic = in_vgpr(kMagicPair);
  const uint32_t row_bytes = uint32_t(uni(P.K)) >> 1;
  const uint32_t row_groups = uint32_t(uni(P.K)) >> 6;
  const uint32_t c0 = uint32_t(li);
  const uint32_t nrows = uint32_t(uni(P.rows));
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(uni_ptr(P.codes), uint64_t(nrows) * row_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(uni_ptr(P.scales), uint64_t(nrows) * row_groups * 2);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(uni_ptr(P.biases), uint64_t(nrows) * row_groups * 2);
  uint32_t u = uint32_t(p - seg_begin);
  RowBuf<CPL> buf;
  {
    bool valid;
    const uint32_t r = unit_row<SWIGLU>(P, u, slot, &valid);
    load_unit<CPL>(buf, cr, sr, br, valid ? r : 0u, row_bytes, row_groups, c0);
  }
  before_x();
  uint32_t xp[CPL][16];
  float xs[CPL];
  if constexpr (LDS_X) x_from_lds<CPL>(xp, xs, xl, c0);
  else load_x<CPL>(xp, xs, make_rsrc(uni_ptr(P.x), uint64_t(uni(P.K)) * 2), c0);
  constexpr int64_t W = kWavesPerBlockSingle;  // the block's waves take its positions in turn
  for (; p < end; p += W, u += uint32_t(W)) {
    const float v = slot_reduce<LPR>(unit_partial<CPL>(buf, xp, xs, magic));
    if (p + W < end) {
      bool valid;
      const uint32_t r = unit_row<SWIGLU>(P, u + uint32_t(W), slot, &valid);
      load_unit<CPL>(buf, cr, sr, br, valid ? r : 0u, row_bytes, row_groups, c0);
    }
    bool valid;
    const uint32_t r = unit_row<SWIGLU>(P, u, slot, &valid);
    if constexpr (SWIGLU) {
      const float up = __shfl_xor(v, 32);
      if (valid && slot == 0 && result_lane) store_out(P.out0, u, silu_times(v, up), P.f32_out);
    } else {
      if (valid && result_lane) store_qkv(P, r, P.lin_bias ? v + bf16_bits_to_f32(P.lin_bias[r]) : v);
    }
  }
  return p;
}

// Where a launch's projections come from.  TableSrc: the plan's tables in device memory
// (restrict-qualified kernel parameters, so that their loads are scalar loads).  InlineSrc:
// a launch of at most kInlineProjs projections carries them in its kernel arguments, which
// saves the dependent table reads before a wave's first weight request.  Segment i of a
// launch is its i-th projection; begin(i) its first position, begin(n_seg) the launch's
// position count.
struct TableSrc {
  const Proj* __restrict__ projs;
  const Seg* __restrict__ segs;
  const BlockSegs* __restrict__ blocks;
  __device__ __forceinline__ const Proj& proj(int si) const { return projs[uni(segs[si].proj)]; }
  __device__ __forceinline__ int64_t begin(int si) const { return segs[si].begin; }
  // segments of the block's first and last positions (positions [p0, p1), p0 < p1)
  __device__ __forceinline__ int first_seg(int64_t) const { return uni(blocks[blockIdx.x].first); }
  __device__ __forceinline__ int last_seg(int64_t) const { return uni(blocks[blockIdx.x].last); }
};

struct InlineSrc {
  const InlineLaunch& L;
  __device__ __forceinline__ const Proj& proj(int si) const { return L.projs[si]; }
  __device__ __forceinline__ int64_t begin(int si) const { return L.begin[si]; }
  __device__ __forceinline__ int seg_of(int64_t q) const {
    int s = 0;
#pragma unroll
    for (int j = 1; j < kInlineProjs; ++j)
      if (j < L.n_seg && L.begin[j] <= q) s = j;
    return s;
  }
  __device__ __forceinline__ int first_seg(int64_t p0) const { return seg_of(p0); }
  __device__ __forceinline__ int last_seg(int64_t p1) const { return seg_of(p1 - 1); }
};

// One single-slice launch: the positions spread evenly over the grid's blocks in contiguous
// ranges (`per` per wave, the first `extra` waves one more, summed over the block's waves),
// which the block's 4 waves take in turn (wave w: the range's positions w, w + 4, ...; at any
// time the block reads 4 adjacent row units: measured 0.3-0.5 % faster than a contiguous
// range per wave, on the 14B and the 24B steps).  LDS_X: the block first stages, once,
// the activations of the (at most two) projections its waves start and end in, and the
// planner takes this variant only where no block's range reaches a third activation vector;
// else every wave reads its activations from memory at each projection it enters.  (One
// kernel with both paths needs more registers than either.)
template <bool LDS_X, typename Src>
__device__ __forceinline__ void single_body(const Src& src, int64_t per, int64_t extra) {
  __shared__ __attribute__((aligned(16))) uint32_t xl[LDS_X ? 2 : 1][LDS_X ? kXWords : 4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto first_of = [&](int64_t gw) { return gw * per + (gw < extra ? gw : extra); };
  int64_t p = uni64(first_of(int64_t(blockIdx.x) * kWavesPerBlockSingle)) + wave;
  const int64_t pend = uni64(first_of(int64_t(blockIdx.x + 1) * kWavesPerBlockSingle));
  const int64_t bp0 = first_of(int64_t(blockIdx.x) * kWavesPerBlockSingle);
  const int64_t bp1 = first_of(int64_t(blockIdx.x + 1) * kWavesPerBlockSingle);
  // the segments of the block's first and last positions (the projections whose
  // activations the block stages, LDS_X), staged once by the whole block while each wave's
  // first weights are on their way
  const int sa = bp0 < bp1 ? src.first_seg(bp0) : 0;
  const int sb = bp0 < bp1 ? src.last_seg(bp1) : 0;
  bool staged = !LDS_X;
  auto stage = [&]() {
    if constexpr (LDS_X) {
      if (staged) return;
      staged = true;
      if (bp0 < bp1) {
        const Proj& A = src.proj(sa);
        const uint16_t* ax = uni_ptr(A.x);
        const int ak = uni(A.K);
        stage_x(xl[0], ax, ak, uni(A.cpl));
        const Proj& B = src.proj(sb);
        const uint16_t* bx = uni_ptr(B.x);
        const int bk = uni(B.K);
        if (sb != sa && (bx != ax || bk != ak)) stage_x(xl[LDS_X ? 1 : 0], bx, bk, uni(B.cpl));
      }
      __syncthreads();
    }
  };
  int si = sa;
  while (p < pend) {
    while (src.begin(si + 1) <= p) ++si;
    si = uni(si);
    const Proj P = src.proj(si);
    const int64_t b = uni64(src.begin(si));
    const int64_t e = uni64(src.begin(si + 1) < pend ? src.begin(si + 1) : pend);
    const uint32_t* x = nullptr;
    if constexpr (LDS_X) {
      const Proj& A = src.proj(sa);
      x = (uni_ptr(P.x) == uni_ptr(A.x) && uni(P.K) == uni(A.K)) ? xl[0] : xl[LDS_X ? 1 : 0];
    }
    const bool sw = P.epi == EPI_SWIGLU;
    switch (P.cpl * 2 + (sw ? 1 : 0)) {
#define QMM_STEP_CASE(C)                                                              \
  case C * 2 + 0: p = run_single<C, false, LDS_X>(P, p, b, e, x, stage); break;     \
  case C * 2 + 1: p = run_single<C, true, LDS_X>(P, p, b, e, x, stage); break;
      QMM_STEP_CASE(1)
      QMM_STEP_CASE(2)
      QMM_STEP_CASE(3)
      QMM_STEP_CASE(4)
      QMM_STEP_CASE(5)
#undef QMM_STEP_CASE
      default: p = e; break;  // not planned (the planner only takes 1 <= cpl <= 5)
    }
  }
  stage();  // a wave with no positions still takes its part in the staging and its barrier
}

template <bool LDS_X>
__global__ void __launch_bounds__(64 * kWavesPerBlockSingle, 3)
    gemv_step_single_kernel(const Proj* __restrict__ projs, const Seg* __restrict__ segs,
                            const BlockSegs* __restrict__ blocks, int64_t per, int64_t extra) {
  single_body<LDS_X>(TableSrc{projs, segs, blocks}, per, extra);
}

template <bool LDS_X>
__global__ void __launch_bounds__(64 * kWavesPerBlockSingle, 3)
    gemv_step_single_inline_kernel(const InlineLaunch L, int64_t per, int64_t extra) {
  single_body<LDS_X>(InlineSrc{L}, per, extra);
}

// ---- K-split launches (K > 5120) -------------------------------------------------------------

// The block's units [u, uend) of one projection (the block's waves are its K slices); `parity`
// counts the block's units across projections for the double-buffered partial sums.
template <int CPL, bool SWIGLU, int KS>
__device__ __forceinline__ void run_split(const Proj P, int64_t u0, int64_t uend, float (*red)[KS][2], int& parity) {
  const int lane = threadIdx.x & 63;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane / LPR;
  const int li = lane % LPR;
  const bool result_lane = lane == slot_result_lane<LPR>(slot);
  const uint32_t magic = in_vgpr(kMagicPair);
  const uint32_t row_bytes = uint32_t(uni(P.K)) >> 1;
  const uint32_t row_groups = uint32_t(uni(P.K)) >> 6;
  const uint32_t c0 = uint32_t(ks * (LPR * CPL) + li);
  const uint32_t nrows = uint32_t(uni(P.rows));
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(uni_ptr(P.codes), uint64_t(nrows) * row_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(uni_ptr(P.scales), uint64_t(nrows) * row_groups * 2);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(uni_ptr(P.biases), uint64_t(nrows) * row_groups * 2);
  uint32_t u = uint32_t(u0);
  RowBuf<CPL> buf;
  {
    bool valid;
    const uint32_t r = unit_row<SWIGLU>(P, u, slot, &valid);
    load_unit<CPL>(buf, cr, sr, br, valid ? r : 0u, row_bytes, row_groups, c0);
  }
  uint32_t xp[CPL][16];
  float xs[CPL];
  load_x<CPL>(xp, xs, make_rsrc(uni_ptr(P.x), uint64_t(uni(P.K)) * 2), c0);
  for (; u < uint32_t(uend); ++u) {
    const float v = slot_reduce<LPR>(unit_partial<CPL>(buf, xp, xs, magic));
    if (u + 1 < uint32_t(uend)) {
      bool valid;
      const uint32_t r = unit_row<SWIGLU>(P, u + 1, slot, &valid);
      load_unit<CPL>(buf, cr, sr, br, valid ? r : 0u, row_bytes, row_groups, c0);
    }
    // double-buffered by the block's unit parity: the next write to this buffer comes after
    // the next unit's barrier, which wave 0 reaches only after reading this one
    float (*rb)[2] = red[parity & 1];
    if (result_lane) rb[ks][slot] = v;
    __syncthreads();
    if (ks == 0) {
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < KS; ++j) t += rb[j][slot];
      bool valid;
      const uint32_t r = unit_row<SWIGLU>(P, u, slot, &valid);
      if constexpr (SWIGLU) {
        const float up = __shfl_xor(t, 32);
        if (valid && slot == 0 && result_lane) store_out(P.out0, u, silu_times(t, up), P.f32_out);
      } else {
        if (valid && result_lane) store_qkv(P, r, P.lin_bias ? t + bf16_bits_to_f32(P.lin_bias[r]) : t);
      }
    }
    ++parity;
  }
}

// One K-split launch: blocks of KS waves, the launch's units spread evenly over the blocks in
// contiguous ranges.  WIDE: the projections with 5 chunks per lane (8 waves, 32768 < K <=
// 40960), kept apart because they take more registers than the rest.
template <int KS, bool WIDE, typename Src>
__device__ __forceinline__ void split_body(const Src& src, int64_t per, int64_t extra) {
  __shared__ float red[2][KS][2];
  const int64_t g = blockIdx.x;
  int64_t p = g * per + (g < extra ? g : extra);
  const int64_t pend = p + per + (g < extra ? 1 : 0);
  int parity = 0;
  int si = p < pend ? src.first_seg(p) : 0;
  while (p < pend) {
    while (src.begin(si + 1) <= p) ++si;
    si = uni(si);
    const Proj P = src.proj(si);
    const int64_t b = uni64(src.begin(si));
    const int64_t e = uni64(src.begin(si + 1) < pend ? src.begin(si + 1) : pend);
    const bool sw = P.epi == EPI_SWIGLU;
    if constexpr (WIDE) {
      if (sw) run_split<5, true, KS>(P, p - b, e - b, red, parity);
      else run_split<5, false, KS>(P, p - b, e - b, red, parity);
    } else {
      switch (P.cpl * 2 + (sw ? 1 : 0)) {
#define QMM_STEP_CASE(C)                                                                        \
  case C * 2 + 0: run_split<C, false, KS>(P, p - b, e - b, red, parity); break;                 \
  case C * 2 + 1: run_split<C, true, KS>(P, p - b, e - b, red, parity); break;
        QMM_STEP_CASE(1)
        QMM_STEP_CASE(2)
        QMM_STEP_CASE(3)
        QMM_STEP_CASE(4)
#undef QMM_STEP_CASE
        default: break;  // not planned
      }
    }
    p = e;
  }
}

template <int KS, bool WIDE>
__global__ void __launch_bounds__(64 * KS)
    gemv_step_split_kernel(const Proj* __restrict__ projs, const Seg* __restrict__ segs,
                           const BlockSegs* __restrict__ blocks, int64_t per, int64_t extra) {
  split_body<KS, WIDE>(TableSrc{projs, segs, blocks}, per, extra);
}

template <int KS, bool WIDE>
__global__ void __launch_bounds__(64 * KS) gemv_step_split_inline_kernel(const InlineLaunch L, int64_t per,
                                                                         int64_t extra) {
  split_body<KS, WIDE>(InlineSrc{L}, per, extra);
}

// ---- host: grouping, plan building and launch -----------------------------------------------

static uint64_t align256(uint64_t b) { return (b + 255) / 256 * 256; }

struct Shape {
  int ks, cpl;
  int64_t units;
};

static bool shape_of(const qmm_step_proj& p, Shape* s) {
  GemvShape g;
  if (!b4::gemv_shape_for_k(p.K, &g) || g.lpr != LPR || g.cpl > kMaxCpl) return false;
  if (g.ksplit != 1 && g.ksplit != 8 && g.ksplit != 16) return false;
  s->ks = g.ksplit;
  s->cpl = g.cpl;
  s->units = p.kind == QMM_STEP_GATE_UP_SWIGLU ? p.rows / 2 : (p.rows + 1) / 2;
  return true;
}

bool shape_ok(const qmm_step_proj& p) {
  Shape s;
  return shape_of(p, &s);
}

static int kind_of(const Shape& s) {
  if (s.ks == 1) return kSingle;
  if (s.ks == 16) return kSplit16;
  return s.cpl == 5 ? kSplit8Wide : kSplit8;
}

// Launches of a step: (level, kind) pairs in increasing order, each with its projections in
// index order.  Returns false if a projection cannot be planned.
struct HostLaunch {
  int level, kind;
  std::vector<int> projs;
};

static bool group(const qmm_step_proj* projs, int n, std::vector<Shape>& sh, std::vector<HostLaunch>& out) {
  sh.resize(n);
  std::vector<int> level(n, 0);
  for (int i = 0; i < n; ++i) {
    if (!shape_of(projs[i], &sh[i])) return false;
    const int j = projs[i].wait_for;
    level[i] = j >= 0 ? level[j] + 1 : 0;
  }
  std::vector<std::pair<int, int>> keys;
  for (int i = 0; i < n; ++i) keys.push_back({level[i], kind_of(sh[i])});
  std::vector<std::pair<int, int>> uniq = keys;
  std::sort(uniq.begin(), uniq.end());
  uniq.erase(std::unique(uniq.begin(), uniq.end()), uniq.end());
  out.clear();
  for (const auto& k : uniq) {
    HostLaunch L{k.first, k.second, {}};
    for (int i = 0; i < n; ++i)
      if (keys[i] == k) L.projs.push_back(i);
    out.push_back(L);
  }
  return true;
}

template <typename Kernel>
static int64_t blocks_per_cu(Kernel k, int threads, int fallback) {
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, threads, 0) != hipSuccess || b < 1) b = fallback;
  return b;
}

// Whether every block of a single-slice launch of `blocks` blocks over these projections sees
// at most two distinct activation vectors (then the LDS variant may run it).
static bool two_x_per_block(const qmm_step_proj* projs, const std::vector<int>& ids, const std::vector<Shape>& sh,
                            int64_t blocks) {
  int64_t total = 0;
  for (int i : ids) total += sh[i].units;
  const int64_t W = blocks * kWavesPerBlockSingle, per = total / W, extra = total % W;
  auto first_of = [&](int64_t gw) { return gw * per + (gw < extra ? gw : extra); };
  size_t k = 0;
  int64_t seg_begin = 0;
  for (int64_t b = 0; b < blocks; ++b) {
    const int64_t b0 = first_of(b * kWavesPerBlockSingle), b1 = first_of((b + 1) * kWavesPerBlockSingle);
    if (b0 >= b1) continue;
    while (seg_begin + sh[ids[k]].units <= b0) seg_begin += sh[ids[k++]].units;
    const qmm_step_proj& A = projs[ids[k]];
    size_t j = k;
    int64_t sj = seg_begin;
    while (sj + sh[ids[j]].units <= b1 - 1) sj += sh[ids[j++]].units;
    const qmm_step_proj& B = projs[ids[j]];
    for (size_t m = k + 1; m < j; ++m) {
      const qmm_step_proj& Q = projs[ids[m]];
      const bool is_a = Q.x == A.x && Q.K == A.K, is_b = Q.x == B.x && Q.K == B.K;
      if (!is_a && !is_b) return false;
    }
  }
  return true;
}

// Grid of each launch and, for single-slice launches, whether the LDS variant runs it and the
// dynamic LDS that holds it to two blocks per CU (0: as many as the registers allow); the same
// at planning and at every run (the plan's per-block tables are for this grid).
struct Geometry {
  int64_t units, blocks;
  bool lds;
  size_t pad;
};

// Long single-slice launches run two blocks (8 waves) per CU instead of three: measured on
// MI355X with QKV + gate+up of L 24B-shaped layers per launch (K = 5120), three blocks per CU
// are faster up to 412 MB per launch (206 MB: 41.9 against 43.5-44.3 us), two from 826 MB on
// (137-139 against 142 us; 8.26 GB: 1.263 against 1.327 ms, 6.54 against 6.22 TB/s).  The
// switch is at kLongUnitsPerWave positions per wave at three blocks per CU (~560 MB at K =
// 5120); the 14B-shaped step (100 MB, ~6 per wave) keeps three.
constexpr int64_t kLongUnitsPerWave = 32;
constexpr size_t kLongBlockLds = 64 * 1024;  // a block's LDS with the padding: 2 per CU fit, 3 do not

// Dynamic LDS that makes a block of kernel k take kLongBlockLds, or 0 if that does not leave
// exactly two blocks per CU (then the launch keeps its register-bound occupancy).
template <typename Kernel>
static size_t long_pad(Kernel k) {
  hipFuncAttributes at{};
  if (hipFuncGetAttributes(&at, reinterpret_cast<const void*>(k)) != hipSuccess || at.sharedSizeBytes >= kLongBlockLds)
    return 0;
  const size_t pad = kLongBlockLds - at.sharedSizeBytes;
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, 64 * kWavesPerBlockSingle, pad) != hipSuccess || b != 2)
    return 0;
  return pad;
}

static std::vector<Geometry> geometry(const qmm_step_proj* projs, const std::vector<Shape>& sh,
                                      const std::vector<HostLaunch>& launches) {
  static const int64_t bpc_lds = blocks_per_cu(gemv_step_single_kernel<true>, 64 * kWavesPerBlockSingle, 3);
  static const int64_t bpc_mem = blocks_per_cu(gemv_step_single_kernel<false>, 64 * kWavesPerBlockSingle, 3);
  static const int64_t bpc_s8 = blocks_per_cu(gemv_step_split_kernel<8, false>, 512, 2);
  static const int64_t bpc_s8w = blocks_per_cu(gemv_step_split_kernel<8, true>, 512, 1);
  static const int64_t bpc_s16 = blocks_per_cu(gemv_step_split_kernel<16, false>, 1024, 1);
  static const size_t pad_lds = long_pad(gemv_step_single_kernel<true>);
  static const size_t pad_mem = long_pad(gemv_step_single_kernel<false>);
  static const size_t pad_lds_in = long_pad(gemv_step_single_inline_kernel<true>);
  static const size_t pad_mem_in = long_pad(gemv_step_single_inline_kernel<false>);
  const int64_t cus = device_cus();
  std::vector<Geometry> g(launches.size());
  for (size_t l = 0; l < launches.size(); ++l) {
    int64_t units = 0;
    for (int i : launches[l].projs) units += sh[i].units;
    g[l].units = units;
    g[l].lds = false;
    g[l].pad = 0;
    const int kind = launches[l].kind;
    if (kind == kSingle) {
      // every wave of the grid resident at once, but no more waves than positions; long
      // launches two blocks per CU (the padding holds them there)
      const int64_t need = (units + kWavesPerBlockSingle - 1) / kWavesPerBlockSingle;
      const bool inl = launches[l].projs.size() <= size_t(kInlineProjs);
      const bool lng = units >= kLongUnitsPerWave * cus * bpc_lds * kWavesPerBlockSingle;
      const size_t pl = lng ? (inl ? pad_lds_in : pad_lds) : 0, pm = lng ? (inl ? pad_mem_in : pad_mem) : 0;
      int64_t blocks = std::min(cus * (pl ? 2 : bpc_lds), need);
      g[l].lds = two_x_per_block(projs, launches[l].projs, sh, blocks);
      if (g[l].lds) {
        g[l].pad = pl;
      } else {
        blocks = std::min(cus * (pm ? 2 : bpc_mem), need);
        g[l].pad = pm;
      }
      g[l].blocks = blocks;
    } else {
      const int64_t bpc = kind == kSplit8 ? bpc_s8 : (kind == kSplit8Wide ? bpc_s8w : bpc_s16);
      g[l].blocks = std::min(cus * bpc, units);
    }
  }
  return g;
}

struct Layout {
  uint64_t proj_off, launch_off, seg_off, blk_off, bytes;
};

static Layout layout_of(int n, const std::vector<HostLaunch>& launches, const std::vector<Geometry>& g) {
  Layout L;
  uint64_t off = align256(sizeof(Header));
  L.proj_off = off;
  off += align256(uint64_t(n) * sizeof(Proj));
  L.launch_off = off;
  off += align256(uint64_t(launches.size()) * sizeof(Launch));
  L.seg_off = off;
  off += align256(uint64_t(n + launches.size()) * sizeof(Seg));
  L.blk_off = off;
  uint64_t nb = 0;
  for (const Geometry& x : g) nb += uint64_t(x.blocks);
  off += align256(nb * sizeof(BlockSegs));
  L.bytes = off;
  return L;
}

uint64_t plan_bytes(const qmm_step_proj* projs, int n) {
  std::vector<Shape> sh;
  std::vector<HostLaunch> launches;
  if (!group(projs, n, sh, launches)) return 0;
  return layout_of(n, launches, geometry(projs, sh, launches)).bytes;
}

// The device record of a projection (a plain projection stores through the QKV routing with
// every row in the first part).
static void fill_proj(const qmm_step_proj& p, const Shape& sh, Proj& d) {
  const bool qkv = p.kind == QMM_STEP_QKV;
  d.x = p.x;
  d.codes = p.codes;
  d.scales = p.scales;
  d.biases = p.biases;
  d.lin_bias = p.lin_bias;
  d.out0 = p.out0;
  d.out1 = qkv ? p.out1 : nullptr;
  d.out2 = qkv ? p.out2 : nullptr;
  d.K = int32_t(p.K);
  d.rows = int32_t(p.rows);
  d.q_out = int32_t(qkv ? p.q_out : p.rows);
  d.kv_out = int32_t(qkv ? p.kv_out : 0);
  d.I = int32_t(p.rows / 2);
  d.epi = p.kind == QMM_STEP_GATE_UP_SWIGLU ? EPI_SWIGLU : EPI_QKV;
  d.f32_out = p.out_dtype == QMM_OUT_F32;
  d.ks = sh.ks;
  d.cpl = sh.cpl;
  d.units = int32_t(sh.units);
}

int build_and_upload(const qmm_step_proj* projs, int n, void* plan, uint64_t bytes, hipStream_t stream) {
  std::vector<Shape> sh;
  std::vector<HostLaunch> launches;
  if (!group(projs, n, sh, launches)) return QMM_ERR_SHAPE;
  const std::vector<Geometry> geo = geometry(projs, sh, launches);
  const Layout lay = layout_of(n, launches, geo);
  if (lay.bytes > bytes) return QMM_ERR_SHAPE;
  std::vector<char> img(lay.bytes, 0);
  Header* hd = reinterpret_cast<Header*>(img.data());
  hd->magic = kMagic;
  hd->n_proj = n;
  hd->n_launch = int32_t(launches.size());
  hd->proj_off = lay.proj_off;
  hd->launch_off = lay.launch_off;
  hd->seg_off = lay.seg_off;
  hd->blk_off = lay.blk_off;
  hd->bytes = lay.bytes;
  Proj* P = reinterpret_cast<Proj*>(img.data() + lay.proj_off);
  Launch* Lr = reinterpret_cast<Launch*>(img.data() + lay.launch_off);
  Seg* S = reinterpret_cast<Seg*>(img.data() + lay.seg_off);
  BlockSegs* B = reinterpret_cast<BlockSegs*>(img.data() + lay.blk_off);
  for (int i = 0; i < n; ++i) fill_proj(projs[i], sh[i], P[i]);
  int ns = 0;
  int64_t nb = 0;
  for (size_t l = 0; l < launches.size(); ++l) {
    Launch& L = Lr[l];
    L.kind = launches[l].kind;
    L.seg0 = ns;
    L.blocks = int32_t(geo[l].blocks);
    L.blk0 = nb;
    std::vector<int64_t> begins;
    int64_t pos = 0;
    for (int i : launches[l].projs) {
      S[ns].begin = pos;
      S[ns].proj = i;
      begins.push_back(pos);
      ++ns;
      pos += sh[i].units;
    }
    L.n_seg = ns - L.seg0;
    L.total = pos;
    S[ns].begin = pos;  // sentinel
    S[ns].proj = launches[l].projs.back();
    ++ns;
    // the segment (relative to this launch) of each block's first and last position
    const int64_t G = geo[l].blocks;
    const int64_t W = L.kind == kSingle ? G * kWavesPerBlockSingle : G;   // position owners
    const int64_t per = pos / W, extra = pos % W;
    auto first_of = [&](int64_t o) { return o * per + (o < extra ? o : extra); };
    const int64_t owners_per_block = L.kind == kSingle ? kWavesPerBlockSingle : 1;
    auto seg_of = [&](int64_t q) {
      return int32_t(std::upper_bound(begins.begin(), begins.end(), q) - begins.begin() - 1);
    };
    for (int64_t b = 0; b < G; ++b) {
      const int64_t b0 = first_of(b * owners_per_block), b1 = first_of((b + 1) * owners_per_block);
      B[nb + b].first = b0 < b1 ? seg_of(b0) : 0;
      B[nb + b].last = b0 < b1 ? seg_of(b1 - 1) : 0;
    }
    nb += G;
  }
  if (hipMemcpyAsync(plan, img.data(), lay.bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return QMM_ERR_LAUNCH;
  if (hipStreamSynchronize(stream) != hipSuccess) return QMM_ERR_LAUNCH;
  return QMM_OK;
}

int launch(const qmm_step_proj* projs, int n, const void* plan, hipStream_t s) {
  std::vector<Shape> sh;
  std::vector<HostLaunch> launches;
  if (!group(projs, n, sh, launches)) return QMM_ERR_SHAPE;
  const std::vector<Geometry> geo = geometry(projs, sh, launches);
  const Layout lay = layout_of(n, launches, geo);
  const char* pl = static_cast<const char*>(plan);
  int seg0 = 0;
  int64_t blk0 = 0;
  for (size_t l = 0; l < launches.size(); ++l) {
    const dim3 grid{unsigned(geo[l].blocks), 1u, 1u};
    const int kind = launches[l].kind;
    // positions per owner (a wave of a single-slice launch, a block of a K-split one)
    const int64_t owners = kind == kSingle ? geo[l].blocks * kWavesPerBlockSingle : geo[l].blocks;
    const int64_t per = geo[l].units / owners, extra = geo[l].units % owners;
    const std::vector<int>& ids = launches[l].projs;
    if (ids.size() <= size_t(kInlineProjs)) {
      InlineLaunch il{};
      int64_t pos = 0;
      for (size_t j = 0; j < ids.size(); ++j) {
        fill_proj(projs[ids[j]], sh[ids[j]], il.projs[j]);
        il.begin[j] = pos;
        pos += sh[ids[j]].units;
      }
      for (size_t j = ids.size(); j <= size_t(kInlineProjs); ++j) il.begin[j] = pos;
      il.n_seg = int32_t(ids.size());
      if (kind == kSingle) {
        const dim3 block{64u * kWavesPerBlockSingle, 1u, 1u};
        if (geo[l].lds) gemv_step_single_inline_kernel<true><<<grid, block, geo[l].pad, s>>>(il, per, extra);
        else gemv_step_single_inline_kernel<false><<<grid, block, geo[l].pad, s>>>(il, per, extra);
      } else if (kind == kSplit8) {
        gemv_step_split_inline_kernel<8, false><<<grid, dim3{512u, 1u, 1u}, 0, s>>>(il, per, extra);
      } else if (kind == kSplit8Wide) {
        gemv_step_split_inline_kernel<8, true><<<grid, dim3{512u, 1u, 1u}, 0, s>>>(il, per, extra);
      } else {
        gemv_step_split_inline_kernel<16, false><<<grid, dim3{1024u, 1u, 1u}, 0, s>>>(il, per, extra);
      }
    } else {
      const Proj* pj = reinterpret_cast<const Proj*>(pl + lay.proj_off);
      const Seg* sg = reinterpret_cast<const Seg*>(pl + lay.seg_off) + seg0;
      const BlockSegs* bk = reinterpret_cast<const BlockSegs*>(pl + lay.blk_off) + blk0;
      if (kind == kSingle) {
        const dim3 block{64u * kWavesPerBlockSingle, 1u, 1u};
        if (geo[l].lds) gemv_step_single_kernel<true><<<grid, block, geo[l].pad, s>>>(pj, sg, bk, per, extra);
        else gemv_step_single_kernel<false><<<grid, block, geo[l].pad, s>>>(pj, sg, bk, per, extra);
      } else if (kind == kSplit8) {
        gemv_step_split_kernel<8, false><<<grid, dim3{512u, 1u, 1u}, 0, s>>>(pj, sg, bk, per, extra);
      } else if (kind == kSplit8Wide) {
        gemv_step_split_kernel<8, true><<<grid, dim3{512u, 1u, 1u}, 0, s>>>(pj, sg, bk, per, extra);
      } else {
        gemv_step_split_kernel<16, false><<<grid, dim3{1024u, 1u, 1u}, 0, s>>>(pj, sg, bk, per, extra);
      }
    }
    if (hipGetLastError() != hipSuccess) return QMM_ERR_LAUNCH;
    seg0 += int(launches[l].projs.size()) + 1;
    blk0 += geo[l].blocks;
  }
  return QMM_OK;
}

}  // namespace step
}  // namespace qmm
