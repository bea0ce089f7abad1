// Routed experts over a batch of tokens (prefill), the parts around the gathered GEMM:
// bucketing the (token, slot) pairs by expert, zeroing the h of pairs with no expert,
// and the per-token combine of the stage-2 products.  The pages keep the expert grid in
// place and select experts by index ("Four Candles for the Cathedral", what's not in
// this batch); prefill needs the selection the other way round, expert -> tokens, so
// that each expert's weights are streamed once for all of its tokens.
//
// Bucketing is deterministic: a pair's position inside its expert's bucket is the number
// of pairs before it (in pair order token * topk + slot) routed to the same expert.  It
// takes three small kernels: per-chunk expert histograms, one block turning them into
// bucket offsets, chunk bases and the tile table, and per-chunk placement.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int kRouteThreads = 256;   // threads of the count and place blocks (one pair each per pass)
constexpr int kScanThreads = 1024;   // the one block of the scan
constexpr int kMaxChunks = 256;      // routing chunks (blocks of the count and place kernels)
constexpr int kScanBatch = 16;       // chunks up to which a scan thread takes a whole expert row
constexpr int kWaveBatch = 8;        // experts a scan wave loads at once above that

static __device__ __forceinline__ bool routed(int32_t e, int E) { return e >= 0 && e < E; }

// Pairs per chunk: a multiple of kRouteThreads, at most kMaxChunks chunks.
static inline int64_t route_chunk(int64_t P) {
  const int64_t per = (P + kMaxChunks - 1) / kMaxChunks;
  const int64_t cs = (per + kRouteThreads - 1) / kRouteThreads * kRouteThreads;
  return cs < kRouteThreads ? kRouteThreads : cs;
}

// counts[e][c] = pairs of chunk c routed to expert e.
__global__ void __launch_bounds__(kRouteThreads) moe_route_count(const int32_t* __restrict__ ids, int64_t P,
                                                                 int64_t cs, int E, int chunks,
                                                                 int32_t* __restrict__ counts) {
  __shared__ int cnt[kMaxExpertsPrefill];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * cs;
  const int64_t end = min(base + cs, P);
  for (int64_t i = base + threadIdx.x; i < end; i += kRouteThreads) {
    const int32_t e = ids[i];
    if (routed(e, E)) atomicAdd(&cnt[e], 1);  // counts only: the order of the adds does not matter
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) counts[int64_t(e) * chunks + blockIdx.x] = cnt[e];
}

// Exclusive prefix sum over the block of one value per thread (kScanThreads threads);
// returns the thread's prefix and sets *total.
static __device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[kScanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    const int ws = wsum[w];
    before += w < wave ? ws : 0;
    all += ws;
  }
  __syncthreads();  // wsum may be reused by the next call
  *total = all;
  return before + inc - v;
}

// One block.  (1) For each expert (a thread each up to kScanBatch chunks, else a wave
// each): counts[e][c] becomes the exclusive prefix over chunks, and the expert's total is
// kept.
// (2) Over the experts: bucket offsets (prefix of the totals), then the tile table: expert
// e's bucket is cut into tiles of `bm` pairs, written at the prefix of the tile counts.
__global__ void __launch_bounds__(kScanThreads) moe_route_scan(int32_t* __restrict__ counts, int chunks, int E,
                                                               int bm, int32_t* __restrict__ hdr,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ tiles) {
  __shared__ int tot[kMaxExpertsPrefill];
  if (chunks <= kScanBatch) {
    // few chunks: one thread per expert, a serial exclusive prefix over its row (all of
    // the row's loads in flight at once; indices clamped into the row, so no branches)
    for (int e = threadIdx.x; e < E; e += kScanThreads) {
      int32_t* row = counts + int64_t(e) * chunks;
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = row[j < chunks ? j : chunks - 1];
      int run = 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (j < chunks) {
          row[j] = run;
          run += v[j];
        }
      }
      tot[e] = run;
    }
  } else {
    // many chunks: a wave per expert (64 chunks per pass, a shuffle scan), kWaveBatch
    // experts' loads issued together so that a wave waits once per batch
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int kWaves = kScanThreads / 64;
    for (int e0 = wave * kWaveBatch; e0 < E; e0 += kWaves * kWaveBatch) {
      int carry[kWaveBatch];
#pragma unroll
      for (int j = 0; j < kWaveBatch; ++j) carry[j] = 0;
      for (int c0 = 0; c0 < chunks; c0 += 64) {
        const int c = c0 + lane;
        const int cc = c < chunks ? c : chunks - 1;
        int v[kWaveBatch], ex[kWaveBatch];
#pragma unroll
        for (int j = 0; j < kWaveBatch; ++j) v[j] = counts[int64_t(e0 + j < E ? e0 + j : E - 1) * chunks + cc];
#pragma unroll
        for (int j = 0; j < kWaveBatch; ++j) {
          const int vj = c < chunks && e0 + j < E ? v[j] : 0;
          int inc = vj;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(inc, d, 64);
            if (lane >= d) inc += u;
          }
          ex[j] = carry[j] + inc - vj;
          carry[j] += __shfl(inc, 63, 64);
        }
#pragma unroll
        for (int j = 0; j < kWaveBatch; ++j)
          if (c < chunks && e0 + j < E) counts[int64_t(e0 + j) * chunks + c] = ex[j];
      }
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kWaveBatch; ++j)
          if (e0 + j < E) tot[e0 + j] = carry[j];
      }
    }
  }
  __syncthreads();
  // each thread takes kPer consecutive experts
  constexpr int kPer = kMaxExpertsPrefill / kScanThreads;
  const int e0 = threadIdx.x * kPer;
  int n_sum = 0, t_sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = e0 + j;
    const int n = e < E ? tot[e] : 0;
    n_sum += n;
    t_sum += (n + bm - 1) / bm;
  }
  int n_all, t_all;
  int off = block_exclusive_scan(n_sum, &n_all);
  int tix = block_exclusive_scan(t_sum, &t_all);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = e0 + j;
    if (e >= E) break;
    const int n = tot[e];
    offsets[e] = off;
    for (int s = 0; s < n; s += bm) {
      tiles[2 * tix] = e;
      tiles[2 * tix + 1] = off + s;
      ++tix;
    }
    off += n;
  }
  if (threadIdx.x == 0) {
    offsets[E] = n_all;
    hdr[0] = t_all;
    hdr[1] = n_all;
  }
}

// Places the pairs of chunk c: pair i routed to e goes to offsets[e] + counts[e][c] + (pairs
// of the chunk before i routed to e).  The chunk is taken kRouteThreads pairs at a time; a
// running count per expert carries over between passes.
__global__ void __launch_bounds__(kRouteThreads) moe_route_place(const int32_t* __restrict__ ids, int64_t P,
                                                                 int64_t cs, int E, int chunks,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ pairs) {
  __shared__ int run[kMaxExpertsPrefill];
  __shared__ int32_t sid[kRouteThreads];
  for (int e = threadIdx.x; e < E; e += kRouteThreads)
    run[e] = offsets[e] + counts[int64_t(e) * chunks + blockIdx.x];
  const int64_t base = int64_t(blockIdx.x) * cs;
  const int64_t end = min(base + cs, P);
  const int t = threadIdx.x;
  for (int64_t b = base; b < end; b += kRouteThreads) {
    const int64_t i = b + t;
    const int32_t e = i < end ? ids[i] : -1;
    sid[t] = e;
    __syncthreads();  // sid written; run holds the counts before this pass
    const bool ok = routed(e, E);
    if (ok) {
      int rank = 0;
      for (int j = 0; j < t; ++j) rank += sid[j] == e;
      pairs[run[e] + rank] = int32_t(i);
    }
    __syncthreads();  // every thread has read run and sid
    if (ok) atomicAdd(&run[e], 1);
  }
}

// h of the pairs with no expert is zero (the gathered GEMM writes routed pairs only):
// one thread per pair, which clears its row when the pair has no expert.
__global__ void __launch_bounds__(256) moe_zero_unrouted(const int32_t* ids, int64_t P, int E, void* h, int64_t I,
                                                         int f32) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= P || routed(ids[i], E)) return;
  for (int64_t c = 0; c < I; ++c) store_out(h, i * I + c, 0.f, f32);
}

// y[m, n] = sum over the token's slots k with an expert, in increasing k, of
// z[m*topk + k, n] (z already holds p * (D_e h) in fp32).  A thread adds 4 consecutive
// columns (one 16-byte load per slot) when N is a multiple of 4, else one.
template <bool VEC4>
__global__ void __launch_bounds__(256) moe_combine(const int32_t* ids, int64_t M, int topk, int E, const float* z,
                                                   int64_t N, void* y, int f32) {
  constexpr int W = VEC4 ? 4 : 1;
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    for (int64_t n = int64_t(threadIdx.x) * W; n < N; n += 256 * W) {
      float acc[W] = {};
      for (int k = 0; k < topk; ++k) {
        const int64_t pr = m * topk + k;
        if (!routed(ids[pr], E)) continue;
        if constexpr (VEC4) {
          const float4 v = *reinterpret_cast<const float4*>(z + pr * N + n);
          acc[0] += v.x;
          acc[1] += v.y;
          acc[2] += v.z;
          acc[3] += v.w;
        } else {
          acc[0] += z[pr * N + n];
        }
      }
#pragma unroll
      for (int e = 0; e < W; ++e) store_out(y, m * N + n + e, acc[e], f32);
    }
  }
}

MoeLayout moe_layout(int64_t M, int64_t topk, int64_t E, int64_t out_rows) {
  MoeLayout L;
  L.P = M * topk;
  L.tmax = (L.P + kMoeTileRows - 1) / kMoeTileRows + E;
  L.chunk_pairs = route_chunk(L.P);
  L.chunks = (L.P + L.chunk_pairs - 1) / L.chunk_pairs;
  auto up = [](uint64_t b) { return (b + 255) / 256 * 256; };
  uint64_t o = 0;
  L.hdr = o;      o = up(o + 16);
  L.offsets = o;  o = up(o + uint64_t(E + 1) * 4);
  L.pairs = o;    o = up(o + uint64_t(L.P) * 4);
  L.tiles = o;    o = up(o + uint64_t(L.tmax) * 8);
  L.chunk = o;    o = up(o + uint64_t(L.chunks) * uint64_t(E) * 4);
  L.z = o;        o = up(o + uint64_t(L.P) * uint64_t(out_rows) * 4);
  L.total = o;
  return L;
}

int launch_moe_route(const int32_t* ids, int64_t M, int64_t topk, int64_t E, void* ws, hipStream_t s) {
  const MoeLayout L = moe_layout(M, topk, E, 0);
  char* b = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b + L.chunk);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  const dim3 blk{unsigned(kRouteThreads), 1u, 1u};
  const dim3 grid{unsigned(L.chunks), 1u, 1u};
  moe_route_count<<<grid, blk, 0, s>>>(ids, L.P, L.chunk_pairs, int(E), int(L.chunks), counts);
  moe_route_scan<<<dim3{1u, 1u, 1u}, dim3{unsigned(kScanThreads), 1u, 1u}, 0, s>>>(
      counts, int(L.chunks), int(E), kMoeTileRows, reinterpret_cast<int32_t*>(b + L.hdr), offsets,
      reinterpret_cast<int32_t*>(b + L.tiles));
  moe_route_place<<<grid, blk, 0, s>>>(ids, L.P, L.chunk_pairs, int(E), int(L.chunks), offsets, counts,
                                       reinterpret_cast<int32_t*>(b + L.pairs));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int launch_moe_prefill(int stage, const GemmArgs& g, const int32_t* ids, int64_t M, int64_t topk, int64_t E,
                       const void* ws, void* out, hipStream_t s) {
  const MoeLayout L = moe_layout(M, topk, E, stage == 0 ? 0 : g.N);
  const char* b = static_cast<const char*>(ws);
  GemmArgs a = g;
  a.moe_hdr = reinterpret_cast<const int32_t*>(b + L.hdr);
  a.moe_tiles = reinterpret_cast<const int32_t*>(b + L.tiles);
  a.moe_offsets = reinterpret_cast<const int32_t*>(b + L.offsets);
  a.moe_pairs = reinterpret_cast<const int32_t*>(b + L.pairs);
  const unsigned zb = unsigned((L.P + 255) / 256);
  if (stage == 0) {
    // stage 1: h [P][I] of the routed pairs from the gathered kernel, zeros for the others
    a.out0 = out;
    a.moe_w = nullptr;
    a.moe_div = topk;
    if (int st = launch_moe_gemm(EPI_SWIGLU, a, L.tmax, s)) return st;
    moe_zero_unrouted<<<dim3{zb, 1u, 1u}, dim3{256u, 1u, 1u}, 0, s>>>(ids, L.P, int(E), out, a.I, a.f32_out);
  } else {
    // stage 2: z = p * (D_e h) per routed pair (fp32, workspace), then the per-token sum
    float* z = reinterpret_cast<float*>(const_cast<char*>(b) + L.z);
    const int f32_y = a.f32_out;
    a.out0 = z;
    a.f32_out = 1;
    a.moe_div = 1;
    if (int st = launch_moe_gemm(EPI_LINEAR, a, L.tmax, s)) return st;
    const unsigned mb = unsigned(M < 4096 ? M : 4096);
    if (a.N % 4 == 0)
      moe_combine<true><<<dim3{mb, 1u, 1u}, dim3{256u, 1u, 1u}, 0, s>>>(ids, M, int(topk), int(E), z, a.N, out, f32_y);
    else
      moe_combine<false><<<dim3{mb, 1u, 1u}, dim3{256u, 1u, 1u}, 0, s>>>(ids, M, int(topk), int(E), z, a.N, out, f32_y);
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace qmm
