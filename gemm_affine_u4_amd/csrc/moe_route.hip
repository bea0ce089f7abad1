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

constexpr int kRouteChunk = 1024;   // pairs per routing block
constexpr int kRouteThreads = 256;

static __device__ __forceinline__ bool routed(int32_t e, int E) { return e >= 0 && e < E; }

__global__ void __launch_bounds__(kRouteThreads) moe_route_count(const int32_t* ids, int64_t P, int E,
                                                                 int32_t* chunk_counts) {
  __shared__ int cnt[kMaxExpertsPrefill];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kRouteChunk;
  for (int t = threadIdx.x; t < kRouteChunk; t += kRouteThreads) {
    const int64_t i = base + t;
    if (i < P) {
      const int32_t e = ids[i];
      if (routed(e, E)) atomicAdd(&cnt[e], 1);  // counts only: their order does not matter
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) chunk_counts[int64_t(blockIdx.x) * E + e] = cnt[e];
}

// One block: per expert the total and the chunk prefix (in place), then bucket offsets and
// the tile table (tiles of up to `bm` pairs, expert by expert), then absolute chunk bases.
__global__ void __launch_bounds__(kRouteThreads) moe_route_scan(int32_t* chunk_counts, int chunks, int E, int bm,
                                                                int32_t* hdr, int32_t* offsets, int32_t* tiles) {
  __shared__ int tot[kMaxExpertsPrefill];
  __shared__ int off[kMaxExpertsPrefill];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    int run = 0;
    for (int c = 0; c < chunks; ++c) {
      const int v = chunk_counts[int64_t(c) * E + e];
      chunk_counts[int64_t(c) * E + e] = run;
      run += v;
    }
    tot[e] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0, nt = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = acc;
      offsets[e] = acc;
      for (int s = 0; s < tot[e]; s += bm) {
        tiles[2 * nt] = e;
        tiles[2 * nt + 1] = acc + s;
        ++nt;
      }
      acc += tot[e];
    }
    offsets[E] = acc;
    hdr[0] = nt;
    hdr[1] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads)
    for (int c = 0; c < chunks; ++c) chunk_counts[int64_t(c) * E + e] += off[e];
}

__global__ void __launch_bounds__(kRouteThreads) moe_route_place(const int32_t* ids, int64_t P, int E,
                                                                 const int32_t* chunk_base, int32_t* pairs) {
  __shared__ int32_t sid[kRouteChunk];
  const int64_t base = int64_t(blockIdx.x) * kRouteChunk;
  for (int t = threadIdx.x; t < kRouteChunk; t += kRouteThreads) {
    const int64_t i = base + t;
    sid[t] = i < P ? ids[i] : -1;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < kRouteChunk; t += kRouteThreads) {
    const int32_t e = sid[t];
    if (!routed(e, E)) continue;
    int rank = 0;
    for (int j = 0; j < t; ++j) rank += sid[j] == e;
    pairs[chunk_base[int64_t(blockIdx.x) * E + e] + rank] = int32_t(base + t);
  }
}

// h of the pairs with no expert is zero (the gathered GEMM writes routed pairs only).
__global__ void __launch_bounds__(256) moe_zero_unrouted(const int32_t* ids, int64_t P, int E, void* h, int64_t I,
                                                         int f32) {
  for (int64_t i = blockIdx.x; i < P; i += gridDim.x) {
    if (routed(ids[i], E)) continue;
    for (int64_t c = threadIdx.x; c < I; c += 256) store_out(h, i * I + c, 0.f, f32);
  }
}

// y[m, n] = sum over the token's slots k with an expert, in increasing k, of
// z[m*topk + k, n] (z already holds p * (D_e h) in fp32).
__global__ void __launch_bounds__(256) moe_combine(const int32_t* ids, int64_t M, int topk, int E, const float* z,
                                                   int64_t N, void* y, int f32) {
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    for (int64_t n = threadIdx.x; n < N; n += 256) {
      float acc = 0.f;
      for (int k = 0; k < topk; ++k) {
        const int64_t pr = m * topk + k;
        if (routed(ids[pr], E)) acc += z[pr * N + n];
      }
      store_out(y, m * N + n, acc, f32);
    }
  }
}

MoeLayout moe_layout(int64_t M, int64_t topk, int64_t E, int64_t out_rows) {
  MoeLayout L;
  L.P = M * topk;
  L.tmax = (L.P + kMoeTileRows - 1) / kMoeTileRows + E;
  L.chunks = (L.P + kRouteChunk - 1) / kRouteChunk;
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
  int32_t* chunk = reinterpret_cast<int32_t*>(b + L.chunk);
  const dim3 blk{unsigned(kRouteThreads), 1u, 1u};
  moe_route_count<<<dim3{unsigned(L.chunks), 1u, 1u}, blk, 0, s>>>(ids, L.P, int(E), chunk);
  moe_route_scan<<<dim3{1u, 1u, 1u}, blk, 0, s>>>(chunk, int(L.chunks), int(E), kMoeTileRows,
                                                   reinterpret_cast<int32_t*>(b + L.hdr),
                                                   reinterpret_cast<int32_t*>(b + L.offsets),
                                                   reinterpret_cast<int32_t*>(b + L.tiles));
  moe_route_place<<<dim3{unsigned(L.chunks), 1u, 1u}, blk, 0, s>>>(ids, L.P, int(E), chunk,
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
  const unsigned zb = unsigned(L.P < 4096 ? L.P : 4096);
  if (stage == 0) {
    // stage 1: h [P][I] of the routed pairs from the gathered GEMM, zeros for the others
    a.out0 = out;
    a.moe_w = nullptr;
    a.moe_div = topk;
    if (int st = launch_gemm_moe(EPI_SWIGLU, a, L.tmax, s)) return st;
    moe_zero_unrouted<<<dim3{zb, 1u, 1u}, dim3{256u, 1u, 1u}, 0, s>>>(ids, L.P, int(E), out, a.I, a.f32_out);
  } else {
    // stage 2: z = p * (D_e h) per routed pair (fp32, workspace), then the per-token sum
    float* z = reinterpret_cast<float*>(const_cast<char*>(b) + L.z);
    const int f32_y = a.f32_out;
    a.out0 = z;
    a.f32_out = 1;
    a.moe_div = 1;
    if (int st = launch_gemm_moe(EPI_LINEAR, a, L.tmax, s)) return st;
    const unsigned mb = unsigned(M < 4096 ? M : 4096);
    moe_combine<<<dim3{mb, 1u, 1u}, dim3{256u, 1u, 1u}, 0, s>>>(ids, M, int(topk), int(E), z, a.N, out, f32_y);
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace qmm
