// Routed experts over a batch of tokens (prefill): the two gathered projections of a layer
// (gate+up+SwiGLU, then down) on the matrix cores, weight-stationary.
//
// The pages keep every expert's weights in place in the grid and pick experts by index
// ("Four Candles for the Cathedral", what's not in this batch); prefill is matmul-bound
// ("Sanctum-MLX", latency testing).  After bucketing, an expert of a 35B-A3B-shaped layer
// holds a few dozen (token, slot) pairs, so its weights are large next to its activations:
// the kernel is built so that each weight is read and dequantized exactly once per routing
// tile, and the activations of the tile's pairs are what is shared through LDS.
//
// A block (8 waves) takes one routing tile (up to 96 pairs of one expert) and one slab of
// 256 of the expert's weight rows, and walks K one 64-wide group per step:
//   * each wave owns 32 weight rows and holds them, dequantized, as the A operand of
//     v_mfma_f32_32x32x16_bf16: lane l reads 16 bytes (32 codes) of row l % 32 per step,
//     half l / 32 of the group, and turns them into w = s*q + b in fp32, rounded to bf16
//     (the same weights as the LDS-dequant GEMM), straight into registers;
//   * the tile's activation rows (gathered through the bucket) go global -> LDS directly
//     (buffer_load ... lds) one step ahead, into a ring of two stages, and every wave
//     reads them as the B operands of its multiplies: one 32 x 32 accumulator per 32 pairs.
// Since MFMA lane l pairs k-slot 8 (l / 32) + t of A with the same slot of B, the slots of
// a 16-wide multiply may stand for any 16 inputs of the group, as long as both operands
// agree: multiply j takes inputs 32 h + 8 j .. +7 from the lanes of half h, so a lane's A
// fragment for multiply j is one code word and its B fragment one 16-byte chunk of the row.
// The number of 32-pair blocks of a tile (1..3) is a template parameter of the loop, so the
// multiplies and the loads of a step are fixed and the wait counts are constants.
#include <type_traits>
#include <utility>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace moe_mm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#ifndef QMM_MOE_WAVES
#define QMM_MOE_WAVES 8
#endif
constexpr int kWaves = QMM_MOE_WAVES;          // waves per block (4, 8 or 16)
constexpr int kSlab = 32 * kWaves;             // weight rows per block
static_assert(kWaves == 4 || kWaves == 8 || kWaves == 16, "waves per block");
// activation load instructions per wave and step for a tile of MB blocks of 32 pairs: the
// tile's 4 MB groups of 8 rows spread over the waves (with 8 waves and an odd MB some waves
// also load a group another wave loads, the same bytes into the same slot)
template <int MB>
constexpr int x_loads() { return (4 * MB + kWaves - 1) / kWaves; }
constexpr int kMaxMB = kMoeTileRows / 32;      // 32-pair blocks per routing tile
constexpr int kRow = 64;                       // bf16 per LDS row (one group of one pair)
constexpr int kXcds = 8;
static_assert(kMaxMB >= 1 && kMaxMB <= 4, "one tile is at most 4 blocks of 32 pairs");
#ifndef QMM_MOE_XDIST
#define QMM_MOE_XDIST 1
#endif
#ifndef QMM_MOE_XSTAGES
#define QMM_MOE_XSTAGES 2
#endif
#ifndef QMM_MOE_MIX
#define QMM_MOE_MIX 1
#endif
#ifndef QMM_MOE_SDIST
#define QMM_MOE_SDIST 4
#endif
// Steps ahead at which the activations (through LDS) and the scale and bias chunks (8
// groups, into registers) are requested, and the ring the activations land in.  The codes
// go through LDS too, two steps (64 bytes of a row) at a time, one such chunk ahead.
constexpr int kXDist = QMM_MOE_XDIST;
constexpr int kXStages = QMM_MOE_XSTAGES;
constexpr int kSDist = QMM_MOE_SDIST;
constexpr int kChunk = 8;                   // groups per scale/bias load (16 bytes)
constexpr int kCodeSteps = 2;               // steps per code chunk
constexpr int kCodeRow = 32 * kCodeSteps;   // bytes of one row in a code chunk
constexpr int kCodeBuf = kSlab * kCodeRow;  // bytes per code chunk buffer
// LDS of a block: the activation stages (MB * 4 KB each) and the code chunk ring, whose depth
// depends on the tile: 4 chunks (requested 5-6 steps ahead) where the stages leave room, else
// 3 or 2.
// Waves per block, LDS pool and blocks per CU: 8 waves (256 weight rows), 56 KB and 2 (16
// waves per CU, at most 128 registers each; the smallest pool the largest tile fits, so the
// code ring is 2 chunks deep for tiles of 33-96 pairs and 3 below) measured 10-13 us per
// 35B-A3B layer at 2048 tokens faster than 4 waves (128 rows) with 40 KB and 4 blocks: the
// 8 waves share one copy of the tile's activations per step, and there are half as many
// blocks, each paying its lookup, prologue and epilogue once.  64 and 72 KB pools (deeper
// code rings) measured 2-6 us slower than 56, 80 KB no faster than 4 waves; 16 waves (512
// rows, one block per CU, 88 or 120 KB) 15-30 us slower; with 8 waves, routing tiles of up
// to 128 pairs (64 or 72 KB) 10-20 us and of up to 64 (48 or 56 KB) 5-15 us slower than of
// up to 96.  With 4 waves:
// 40 KB and 4 blocks measured 1-10 us per layer faster than 48 KB and 3 with tiles of up
// to 128 pairs, and 5 blocks of 32 KB (96 registers: spills) slower.
#ifndef QMM_MOE_LDS_KB
#define QMM_MOE_LDS_KB 56
#endif
#ifndef QMM_MOE_BLOCKS_PER_CU
#define QMM_MOE_BLOCKS_PER_CU 2
#endif
constexpr int kLds = QMM_MOE_LDS_KB * 1024;
constexpr int kBlocksPerCU = QMM_MOE_BLOCKS_PER_CU;
// the pair list sits beside the pool, or (when that would cost a block per CU) in the pool,
// read into registers before the pool's first loads
constexpr bool kPairsInPool = (kLds + kMoeTileRows * 4) * kBlocksPerCU > 160 * 1024;
template <int MB>
constexpr int code_chunks() {
  return kXStages * MB * 32 * kRow * 2 + 4 * kCodeBuf <= kLds ? 4
       : kXStages * MB * 32 * kRow * 2 + 3 * kCodeBuf <= kLds ? 3 : 2;
}
static_assert(kXStages > kXDist && kXDist >= 1 && kXDist <= 2, "activation ring");
static_assert(kXStages * kMaxMB * 32 * kRow * 2 + 2 * kCodeBuf <= kLds, "LDS of the largest tile");
static_assert(kSDist >= kXDist && kSDist <= kChunk, "request order the wait counts rely on");
constexpr int gcd_(int a, int b) { return b == 0 ? a : gcd_(b, a % b); }
constexpr int lcm_(int a, int b) { return a / gcd_(a, b) * b; }
// steps until the activation ring, the code buffers and the scale chunks all repeat
constexpr int kUnroll = lcm_(lcm_(kXStages, 4 * kCodeSteps), kChunk);

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Bank-group swizzle of LDS row r: slot c of row r holds the row's 16-byte chunk c ^ swz(r),
// so the 32 rows one operand read spans (at one chunk) hit distinct bank groups.
__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r & 7u) ^ ((r >> 3) & 1u); }

template <int n>
__device__ __forceinline__ float ubyte_f32(uint32_t v) { return float((v >> (8 * n)) & 0xFFu); }

// Wait until at most N of this wave's vector-memory loads are outstanding and its LDS
// reads are done, then meet the other waves (one asm block: the compiler's own barrier
// would wait for the loads requested for later steps too).
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Codes 0..7 of word w (one per nibble, first code in the low nibble) as 8 bf16 weights
// s*q + b (fp32 FMA, exact product, then RNE): one MFMA operand fragment.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float s, float b) {
  const uint32_t lo = in_vgpr(w & 0x0F0F0F0Fu);
  const uint32_t hi = in_vgpr((w >> 4) & 0x0F0F0F0Fu);
  const u32x4_t v = {pack_bf16x2(fmaf(s, ubyte_f32<0>(lo), b), fmaf(s, ubyte_f32<0>(hi), b)),
                     pack_bf16x2(fmaf(s, ubyte_f32<1>(lo), b), fmaf(s, ubyte_f32<1>(hi), b)),
                     pack_bf16x2(fmaf(s, ubyte_f32<2>(lo), b), fmaf(s, ubyte_f32<2>(hi), b)),
                     pack_bf16x2(fmaf(s, ubyte_f32<3>(lo), b), fmaf(s, ubyte_f32<3>(hi), b))};
  return __builtin_bit_cast(bf16x8_t, v);
}

// The same 8 weights from fp16 code pairs: nibbles t and t + 4 of w go into the mantissa of
// the fp16 pair 1024 + q (0x6400 | q, exact), and one v_fma_mix_f32 per code gives
// s * (1024 + q) + (b - 1024 s) in fp32, which is s*q + b rounded once, as above, whenever
// b - 1024 s is exact in fp32 (b = 0 or |b| >= about |s| / 64; otherwise it differs from it
// by at most |s| * 2^-14).  19 VALU ops per 8 codes instead of 23.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8_t dequant8_mix(uint32_t w, float s, float b1024, uint32_t nib, uint32_t magic) {
  f16x2_t d[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) d[t] = __builtin_bit_cast(f16x2_t, ((w >> (4 * t)) & nib) | magic);
  float f[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] = fmaf(s, float(d[k % 4][k / 4]), b1024);
  const u32x4_t v = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Scales and biases of 8 consecutive groups of one row (bf16 pairs).
struct ChunkRegs {
  u32x4_t s, b;
};
// Scale and bias of one group (bf16 bits, zero-extended).
struct GroupRegs {
  uint32_t s, b;
};

// 4 consecutive outputs starting at element idx of dst: one vector store when all exist and
// the address is aligned to it, else element stores.
__device__ __forceinline__ void put4(void* dst, int64_t idx, const float (&v)[4], int nvalid, bool f32) {
  const uintptr_t addr = reinterpret_cast<uintptr_t>(dst) + uintptr_t(idx) * (f32 ? 4u : 2u);
  if (nvalid == 4 && (addr & (f32 ? 15u : 7u)) == 0) {
    if (f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(dst) + idx) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + idx) =
          make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                     f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < nvalid) store_out(dst, idx + e, v[e], f32);
  }
}

// Requests of step t (negative: before step 0), in this order: the activations of step
// t + kXDist (MB wave instructions, 8 rows each), half of the code chunk of steps
// 2 (t/2 + NC - 1) .. +1 (one instruction), then SC8: on chunk steps the scale and bias chunk
// of steps 8c .. 8c+7 (requested kSDist steps before step 8c); otherwise the scale and
// bias of step t + 1.
template <bool SC8>
constexpr bool chunk_step(int t) { return SC8 && ((t + kSDist) % kChunk + kChunk) % kChunk == 0; }
template <bool SC8>
constexpr int tail_loads(int t) { return SC8 ? (chunk_step<SC8>(t) ? 2 : 0) : 2; }
template <int MB, bool SC8>
constexpr int step_loads(int t) { return x_loads<MB>() + 1 + tail_loads<SC8>(t); }
// At the top of step ks (position P in the unrolled loop; P and ks agree modulo 8) its
// activations (requested at step ks - kXDist) and its code chunk (both halves, the later
// one at step 2 floor(ks/2) - 1) must have landed; loads complete in order, so what may
// still be outstanding is what was requested after the later of the two.
template <int MB, bool SC8, int P>
constexpr int wait_count() {
  constexpr int NC = code_chunks<MB>();
  int after_x = 1 + tail_loads<SC8>(P - kXDist);
  for (int u = P - kXDist + 1; u < P; ++u) after_x += step_loads<MB, SC8>(u);
  // chunk c = floor(P/2) is requested at steps 2 (c - NC + 1) and 2 (c - NC + 1) + 1
  const int u0 = 2 * (P >> 1) - 2 * NC + 3;
  int after_c = tail_loads<SC8>(u0);
  for (int u = u0 + 1; u < P; ++u) after_c += step_loads<MB, SC8>(u);
  return after_x < after_c ? after_x : after_c;
}

// Where a block's work sits: its routing tile and weight slab.
struct TileJob {
  int e;                 // expert
  int P;                 // pairs in the tile (1 .. kMoeTileRows)
  int slab;              // weight slab
  const int32_t* pairs;  // the tile's pair indices (LDS)
};

// The tile loop for a tile of MB blocks of 32 pairs.  SC8: the scales and biases are read
// 8 groups (16 bytes) at a time, which needs rows of a multiple of 8 groups (K % 512 == 0)
// for alignment; otherwise one group per step.
template <int EPI, int MB, bool SC8>
__device__ __forceinline__ void tile_body(const GemmArgs& a, const TileJob& jb, unsigned char* lds) {
  constexpr int NC = code_chunks<MB>();
  constexpr int kXStageBytes = MB * 32 * kRow * 2;
  static_assert(kXStages * kXStageBytes + NC * kCodeBuf <= kLds, "LDS of the tile");
  uint16_t* xs_all = reinterpret_cast<uint16_t*>(lds);
  unsigned char* cs_all = lds + kXStages * kXStageBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t K = uint32_t(a.K);
  const int ksteps = int(K >> 6);
  const int last = ksteps - 1;
  const uint32_t groups = K >> 6;
  const int m = lane & 31;  // A row (weight row of the wave) and B column (pair of a block)
  const int h = lane >> 5;  // half of the group this lane's k-slots cover

  // ---- weight rows ------------------------------------------------------------------
  // SwiGLU: the wave's 32 A rows are 16 gate rows and their 16 up rows, A row r being gate
  // (bit 3 of r clear) or up (set) of h index i0 + 8 (r >> 4) + (r & 7); an accumulator's
  // registers 8g + e and 8g + 4 + e (e < 4) then hold gate and up of one index.
  // Linear: A row r is weight row slab*128 + 32 wave + r.  Rows past the end read the last
  // row (their outputs are never stored).
  auto weight_row = [&](int r) -> int64_t {
    if constexpr (EPI == EPI_SWIGLU) {
      int64_t i = int64_t(jb.slab) * (kSlab / 2) + 16 * wave + 8 * (r >> 4) + (r & 7);
      if (i >= a.I) i = a.I - 1;
      return ((r >> 3) & 1) ? a.I + i : i;
    } else {
      const int64_t n = int64_t(jb.slab) * kSlab + 32 * wave + r;
      return n < a.N ? n : a.N - 1;
    }
  };
  const int64_t er = int64_t(jb.e) * a.N;  // first row of the expert in the grid
  const uint64_t nrows = uint64_t(a.N);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.codes + er * (K >> 3), nrows * (K >> 1));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales + er * groups, nrows * groups * 2);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.biases + er * groups, nrows * groups * 2);
  const uint32_t goff = uint32_t(weight_row(m)) * groups * 2u;  // the lane's row's scales

  // Codes: global -> LDS, a chunk of two steps (64 bytes of a row) at a time, into a ring of
  // NC buffers of the block's kSlab rows x 64 bytes.  At step t a wave requests half (rows
  // 16 (t % 2) .. +15 of its 32) of chunk t/2 + NC - 1: lane L takes row 16 (t % 2) + L / 4 and
  // lands in slot L % 4 of it, which holds the row's 16-byte piece (L % 4) ^ cswz(row), so
  // that the 16 rows an operand read spans (at one piece) hit distinct bank groups.  A wave
  // only ever reads its own rows.
  auto cswz = [](uint32_t r) -> uint32_t { return (r >> 2) & 3u; };
  uint32_t cdoff[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 16 * hh + (lane >> 2);
    const uint32_t piece = uint32_t(lane & 3) ^ cswz(uint32_t(32 * wave + r));
    cdoff[hh] = uint32_t(weight_row(r)) * (K >> 1) + piece * 16u;
  }
  auto load_codes = [&](int t) {  // t >= -2 (NC - 1)
    const int hh = t & 1;
    const int c = min((t + 2 * (NC - 1)) >> 1, last >> 1);
    unsigned char* dst = cs_all + (c % NC) * kCodeBuf + (32 * wave + 16 * hh) * kCodeRow;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (__attribute__((address_space(3))) void*)dst, 16, cdoff[hh],
                                             uint32_t(c) * uint32_t(kCodeRow), 0, 0);
  };
  // the lane's 16 bytes of step ks: row 32 wave + m, piece 2 (ks % 2) + h
  const uint32_t crow = uint32_t(32 * wave + m);
  auto read_codes = [&](int ks) -> u32x4_t {
    const uint32_t piece = uint32_t(2 * (ks & 1) + h) ^ cswz(crow);
    return *reinterpret_cast<const u32x4_t*>(cs_all + ((ks >> 1) % NC) * kCodeBuf + crow * kCodeRow + piece * 16u);
  };
  const int last_chunk = int(groups / kChunk) - 1;
  auto load_chunk = [&](ChunkRegs& r, int c) {
    r.s = __builtin_amdgcn_raw_buffer_load_b128(sr, goff + uint32_t(c) * 16u, 0, 0);
    r.b = __builtin_amdgcn_raw_buffer_load_b128(br, goff + uint32_t(c) * 16u, 0, 0);
  };
  auto load_group = [&](GroupRegs& r, int g) {
    r.s = __builtin_amdgcn_raw_buffer_load_b16(sr, goff + uint32_t(g) * 2u, 0, 0);
    r.b = __builtin_amdgcn_raw_buffer_load_b16(br, goff + uint32_t(g) * 2u, 0, 0);
  };

  // ---- the tile's activation rows: global -> LDS ------------------------------------
  // Instruction j (j < x_loads) of wave w fills the LDS rows of group xgroup(w, j): rows
  // 8 group + L / 8, slot L % 8 (lane L lands at byte 16 L), i.e. chunk (L % 8) ^ swz(row)
  // of that pair's row.  Rows past the tile's pairs read its last pair (never stored).
  constexpr int JX = x_loads<MB>();
  auto xgroup = [&](int j) -> int { return kWaves == 4 ? MB * wave + j : (wave + kWaves * j) % (4 * MB); };
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint64_t(a.M) * K * 2);
  uint32_t xoff[JX];
#pragma unroll
  for (int j = 0; j < JX; ++j) {
    const int r = 8 * xgroup(j) + (lane >> 3);
    const int64_t xrow = jb.pairs[min(r, jb.P - 1)] / a.moe_div;
    const uint32_t chunk = uint32_t(lane & 7) ^ swz(uint32_t(r));
    xoff[j] = uint32_t(xrow) * K * 2u + chunk * 16u;
  }
  // the pairs of the lane's output columns, for the epilogue (kept in registers only when
  // the list sits in the pool, which the loads below overwrite)
  int32_t pairs_of[MB];
  if constexpr (kPairsInPool) {
#pragma unroll
    for (int b = 0; b < MB; ++b) pairs_of[b] = jb.pairs[min(32 * b + m, jb.P - 1)];
    __syncthreads();  // every wave has read the list before the pool fills
  }
  auto stage = [&](int p) -> uint16_t* { return xs_all + p * (kXStageBytes / 2); };
  auto load_x = [&](uint16_t* dst, int ks) {
#pragma unroll
    for (int j = 0; j < JX; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (__attribute__((address_space(3))) void*)(dst + 8 * xgroup(j) * kRow), 16, xoff[j],
          uint32_t(ks) * 128u, 0, 0);
  };

  // B operand of multiply j for block b: row 32 b + m, chunk 4 h + j (swz(32 b + m) = swz(m))
  uint32_t boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) boff[j] = uint32_t(m) * kRow + ((uint32_t(4 * h + j) ^ swz(uint32_t(m))) * 8u);

  f32x16_t acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = f32x16_t{};
  const uint32_t nib = in_vgpr(0x000F000Fu), magic = in_vgpr(0x64006400u);

  // Step ks: activations in stage ks % kXStages, codes in code buffer (ks / 2) % NC, scale
  // and bias in chunk `cur` (SC8) or in group set ks % 2.  After the barrier at its top
  // (every wave is done with the previous step) the stage read kXStages - kXDist steps back
  // takes the activations of step ks + kXDist, and the code buffer read by the previous
  // chunk takes half of chunk ks/2 + NC - 1; at the first step of a scale chunk the chunk
  // requested kSDist steps back becomes `cur`.  Requested steps and chunks are clamped to
  // the last one, so every step issues the loads the wait counts assume (the extra copies
  // are never read, or rewrite a buffer with the bytes it already holds).
  ChunkRegs cur, next;
  GroupRegs G[2];
  auto requests = [&](int t, auto p_c) {
    constexpr int P = decltype(p_c)::value;  // t's position modulo kUnroll (t may be < 0)
    if (t + kXDist >= 0) load_x(stage((P + kXDist) % kXStages), min(t + kXDist, last));
    __builtin_amdgcn_sched_barrier(0);  // the wait counts need this order
    if (t >= -2 * (NC - 1)) load_codes(t);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SC8) {
      if constexpr (chunk_step<SC8>(P)) {
        if (t + kSDist >= 0) load_chunk(next, min((t + kSDist) / kChunk, last_chunk));
      }
    } else {
      if (t + 1 >= 0) load_group(G[(P + 1) & 1], min(t + 1, last));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int ks, auto p_c) {
    constexpr int P = decltype(p_c)::value;
    constexpr int kWait = wait_count<MB, SC8, P>();
    wait_loads_barrier<kWait>();
    if constexpr (SC8 && P % kChunk == 0) {
      // taken here and not before, or the compiler may wait for the chunk right after
      // requesting it
      asm volatile("" : "+v"(next.s), "+v"(next.b));
      cur = next;
    }
    const u32x4_t codes = read_codes(ks);
    requests(ks, p_c);
    float s, bb;
    if constexpr (SC8) {
      constexpr int i = P % kChunk;
      const uint32_t sw = cur.s[i / 2], bw = cur.b[i / 2];
      s = __uint_as_float((i & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
      bb = __uint_as_float((i & 1) ? (bw & 0xFFFF0000u) : (bw << 16));
    } else {
      GroupRegs& g = G[P & 1];
      asm volatile("" : "+v"(g.s), "+v"(g.b));
      s = __uint_as_float(g.s << 16);
      bb = __uint_as_float(g.b << 16);
    }
    const uint16_t* xs = stage(P % kXStages);
    // multiply j: its B fragments were read and its A fragment dequantized in phase j - 1
    bf16x8_t xb[2][MB];
    bf16x8_t wa[2];
#pragma unroll
    for (int b = 0; b < MB; ++b) xb[0][b] = *reinterpret_cast<const bf16x8_t*>(xs + 32 * b * kRow + boff[0]);
#if QMM_MOE_MIX
    const float b1024 = fmaf(-1024.f, s, bb);
#define QMM_DEQ(w) dequant8_mix(w, s, b1024, nib, magic)
#else
#define QMM_DEQ(w) dequant8(w, s, bb)
#endif
    wa[0] = QMM_DEQ(codes[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) {
#pragma unroll
        for (int b = 0; b < MB; ++b)
          xb[(j + 1) & 1][b] = *reinterpret_cast<const bf16x8_t*>(xs + 32 * b * kRow + boff[j + 1]);
        wa[(j + 1) & 1] = QMM_DEQ(codes[j + 1]);
      }
#pragma unroll
      for (int b = 0; b < MB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[j & 1], xb[j & 1][b], acc[b], 0, 0, 0);
      // Order inside the phase: the next fragments' LDS reads first (their latency runs
      // under the multiplies), then each multiply followed by a share of the next
      // dequantization (~23 VALU ops), which issues while the multiply executes.
      if (j < 3) {
        __builtin_amdgcn_sched_group_barrier(0x100, MB, 0);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (24 + MB - 1) / MB, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#undef QMM_DEQ
  // Prologue: the requests of the steps before step 0, as those steps would have made them
  // (so the wait counts hold from the first step on).
  constexpr int kLead = (SC8 && kSDist > 2 * (NC - 1)) ? kSDist : 2 * (NC - 1);
  static_for<kLead>([&](auto tc) {
    constexpr int t = decltype(tc)::value - kLead;  // -kLead .. -1
    requests(t, std::integral_constant<int, ((t % kUnroll) + kUnroll) % kUnroll>{});
  });
  int ks = 0;
  for (; ks + kUnroll <= ksteps; ks += kUnroll)
    static_for<kUnroll>([&](auto pc) { step(ks + decltype(pc)::value, pc); });
  static_for<kUnroll - 1>([&](auto pc) {
    if (ks + decltype(pc)::value < ksteps) step(ks + decltype(pc)::value, pc);
  });
  // The copies requested past the last step are never read; without a use the compiler
  // drops those loads, and the wait counts above, which count every step's loads, would no
  // longer cover the activations.  The clamped extra LDS loads still write this block's LDS:
  // let everything land before the block exits.
  if constexpr (SC8) asm volatile("" ::"v"(next.s), "v"(next.b));
  else asm volatile("" ::"v"(G[0].s), "v"(G[0].b), "v"(G[1].s), "v"(G[1].b));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue ---------------------------------------------------------------------
  // Register 4g + e (g < 4, e < 4) of acc[b] in lane l holds A row 8g + 4h + e of the
  // wave against pair 32 b + m of the tile.
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int q = 32 * b + m;
    if (q >= jb.P) continue;
    const int64_t pr = kPairsInPool ? pairs_of[b] : jb.pairs[q];
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int64_t i0 = int64_t(jb.slab) * (kSlab / 2) + 16 * wave + 8 * g + 4 * h;
        if (i0 >= a.I) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = silu_times(acc[b][8 * g + e], acc[b][8 * g + 4 + e]);
        put4(a.out0, pr * a.I + i0, v, int(min<int64_t>(4, a.I - i0)), a.f32_out);
      }
    } else {
      const float sc = a.moe_w ? a.moe_w[pr] : 1.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n0 = int64_t(jb.slab) * kSlab + 32 * wave + 8 * g + 4 * h;
        if (n0 >= a.N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = acc[b][4 * g + e] * sc + ((a.lin_bias && n0 + e < a.N) ? bf16_bits_to_f32(a.lin_bias[n0 + e]) : 0.f);
        put4(a.out0, pr * a.N + n0, v, int(min<int64_t>(4, a.N - n0)), a.f32_out);
      }
    }
  }
}

// The tile loop instance for the tile's number of 32-pair blocks.
template <int EPI, bool SC8>
__device__ __forceinline__ void run_tile(const GemmArgs& a, const TileJob& jb, unsigned char* lds) {
  const int mb = (jb.P + 31) >> 5;
  if (kMaxMB <= 1 || mb <= 1) tile_body<EPI, 1, SC8>(a, jb, lds);
  else if (kMaxMB <= 2 || mb == 2) tile_body<EPI, (kMaxMB < 2 ? 1 : 2), SC8>(a, jb, lds);
  else if (kMaxMB <= 3 || mb == 3) tile_body<EPI, (kMaxMB < 3 ? 1 : 3), SC8>(a, jb, lds);
  else tile_body<EPI, (kMaxMB < 4 ? 1 : 4), SC8>(a, jb, lds);
}

// Stage 1's h of a pair with no expert is zero (tiles write routed pairs only): the blocks
// without a tile take the pairs in turn, block q of nq.
__device__ __forceinline__ void zero_unrouted(const GemmArgs& a, int64_t q, int64_t nq) {
  const int64_t P = a.M * a.moe_div;
  for (int64_t i = q * blockDim.x + threadIdx.x; i < P; i += nq * blockDim.x) {
    const int32_t e = a.moe_ids[i];
    if (e >= 0 && e < a.moe_E) continue;
    for (int64_t c = 0; c < a.I; ++c) store_out(a.out0, i * a.I + c, 0.f, a.f32_out);
  }
}

// Block b runs on XCD b % 8 (blocks go to the XCDs round-robin) and takes tile
// 8 (j / slabs) + b % 8 and slab j % slabs of it, j = b / 8: every slab of a tile on one XCD,
// so the tile's activation rows stay in that XCD's L2, and consecutive tiles on consecutive
// XCDs, so the tiles actually routed (a prefix of the records whose length only the device
// knows) spread over all eight.  The tile is known from the block index alone, so the
// table's length, the record head and the pair indices come in one memory round trip.
template <int EPI>
// (the second bound is the waves per SIMD: kBlocksPerCU blocks of kWaves waves over 4 SIMDs)
__global__ void __launch_bounds__(64 * kWaves, kBlocksPerCU * kWaves / 4) moe_gemm_kernel(GemmArgs a, int64_t slabs) {
  // one LDS object: with a second one beside the pool the compiler waits for the pool's
  // direct-to-LDS loads before every LDS read (vmcnt), which undoes the prefetch
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds + (kPairsInPool ? 0 : kMoeTileRows * 4)];
  int32_t* plist = reinterpret_cast<int32_t*>(lds + (kPairsInPool ? 0 : kLds));
  const int64_t j = blockIdx.x / kXcds;
  const int64_t jt = j / slabs;
  const int64_t tile = jt * kXcds + blockIdx.x % kXcds;
  const int slab = int(j - jt * slabs);
  const int32_t* rec = a.moe_recs + tile * kMoeRecInts;
  const int tiles = a.moe_hdr[0];
  const int e = rec[0];
  const int n = rec[1];
  if (threadIdx.x < kMoeTileRows) plist[threadIdx.x] = rec[kMoeRecHead + threadIdx.x];
  if (tile >= tiles) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int64_t records = int64_t(gridDim.x) / kXcds / slabs * kXcds;
      zero_unrouted(a, (tile - tiles) * slabs + slab, (records - tiles) * slabs);
    }
    return;
  }
  __syncthreads();
  const TileJob jb{e, __builtin_amdgcn_readfirstlane(n), slab, plist};
  if ((a.K >> 6) % kChunk == 0) {
    run_tile<EPI, true>(a, jb, lds);
  } else {
    run_tile<EPI, false>(a, jb, lds);
  }
}

}  // namespace moe_mm

bool moe_gemm_supports(const GemmArgs& a) {
  // group 64, K a whole number of groups, and every buffer offset in 32 bits
  const uint64_t K = uint64_t(a.K);
  return K >= 64 && K % 64 == 0 && uint64_t(a.M) * K * 2u < 0xFFFFFFF0ull &&
         uint64_t(a.N) * K / 2u < 0xFFFFFFF0ull && a.N >= 1;
}

int launch_moe_gemm(int epi, const GemmArgs& a, int64_t m_tiles, hipStream_t s) {
  if (!moe_gemm_supports(a)) return 2;
  const int64_t slabs = epi == EPI_SWIGLU ? (a.I + moe_mm::kSlab / 2 - 1) / (moe_mm::kSlab / 2)
                                          : (a.N + moe_mm::kSlab - 1) / moe_mm::kSlab;
  if (m_tiles % moe_mm::kXcds) return 2;
  const int64_t blocks = m_tiles * slabs;
  if (blocks > 0x7FFFFFFF) return 2;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  const dim3 block{unsigned(64 * moe_mm::kWaves), 1u, 1u};
  if (epi == EPI_SWIGLU) {
    moe_mm::moe_gemm_kernel<EPI_SWIGLU><<<grid, block, 0, s>>>(a, slabs);
  } else if (epi == EPI_LINEAR) {
    moe_mm::moe_gemm_kernel<EPI_LINEAR><<<grid, block, 0, s>>>(a, slabs);
  } else {
    return 5;
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace qmm
