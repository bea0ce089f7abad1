// Routed experts over a batch of tokens (prefill), the parts around the gathered GEMM:
// bucketing the (token, slot) pairs by expert into tile records, and the per-token combine
// of the stage-2 products.  The pages keep the expert grid in place and select experts by
// index ("Four Candles for the Cathedral", what's not in this batch); prefill needs the
// selection the other way round, expert -> tokens, so that each expert's weights are
// streamed once for all of its tokens.
//
// Expert e's bucket (its n_e pairs) fills tiles tb(e) .. tb(e) + ceil(n_e / 128) - 1, tb the
// prefix of the tile counts over the experts; bucket position pos lands in tile
// tb(e) + pos / 128, slot pos % 128, and each tile's record carries its expert, pair count
// and pair indices, so that a GEMM block reads all it needs about its tile in one memory
// round trip.  Up to 16384 pairs and 1024 experts one block does it all in one launch,
// in LDS; above that three kernels (per-chunk histograms, one block for the prefixes and
// record heads, per-chunk placement) do, with positions in pair order (token * topk +
// slot) inside a bucket.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int kRouteThreads = 256;   // threads of the count and place blocks (one pair each per pass)
constexpr int kScanThreads = 1024;   // the one block of the scan
constexpr int kMaxChunks = 256;      // routing chunks (blocks of the count and place kernels)
constexpr int kScanBatch = 16;       // chunks up to which a scan thread takes a whole expert row
constexpr int kWaveBatch = 8;        // experts a scan wave loads at once above that
// One block does the whole routing up to kOneMaxP pairs and kOneMaxE experts.
constexpr int kOneMaxP = 16384;
constexpr int kOneMaxE = kScanThreads;
constexpr int kOneRegs = kOneMaxP / kScanThreads;              // pairs per thread (in registers)
constexpr int kOneMaxTiles = kOneMaxP / kMoeTileRows + kOneMaxE;  // fewer tiles than this
constexpr int kCopyBatch = 8;                                   // slots per thread per copy-out pass
static_assert(kOneMaxP < (1 << 16) && kOneMaxTiles < (1 << 15), "packed prefixes");

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

// The heads of expert e's records: tiles tb .. tb + ceil(n / kMoeTileRows) - 1, each with
// the expert and its number of pairs.
static __device__ void write_heads(int32_t* __restrict__ recs, int e, int n, int tb) {
  for (int j = 0; j * kMoeTileRows < n; ++j)
    *reinterpret_cast<int4*>(recs + int64_t(tb + j) * kMoeRecInts) = make_int4(e, min(kMoeTileRows, n - j * kMoeTileRows), 0, 0);
}

// One block.  (1) For each expert (a thread each up to kScanBatch chunks, else a wave
// each): counts[e][c] becomes the exclusive prefix over chunks, and the expert's total is
// kept.
// (2) Over the experts: the first tile of each expert's records (prefix of the tile
// counts) and the record heads.
__global__ void __launch_bounds__(kScanThreads) moe_route_scan(int32_t* __restrict__ counts, int chunks, int E,
                                                               int32_t* __restrict__ hdr,
                                                               int32_t* __restrict__ tbase,
                                                               int32_t* __restrict__ recs) {
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
    t_sum += (n + kMoeTileRows - 1) / kMoeTileRows;
  }
  int n_all, t_all;
  block_exclusive_scan(n_sum, &n_all);
  int tix = block_exclusive_scan(t_sum, &t_all);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = e0 + j;
    if (e >= E) break;
    const int n = tot[e];
    tbase[e] = tix;
    write_heads(recs, e, n, tix);
    tix += (n + kMoeTileRows - 1) / kMoeTileRows;
  }
  if (threadIdx.x == 0) {
    hdr[0] = t_all;
    hdr[1] = n_all;
  }
}

// Places the pairs of chunk c: pair i routed to e takes bucket position counts[e][c] + (pairs
// of the chunk before i routed to e).  The chunk is taken kRouteThreads pairs at a time; a
// running count per expert carries over between passes.
__global__ void __launch_bounds__(kRouteThreads) moe_route_place(const int32_t* __restrict__ ids, int64_t P,
                                                                 int64_t cs, int E, int chunks,
                                                                 const int32_t* __restrict__ tbase,
                                                                 const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ recs) {
  __shared__ int run[kMaxExpertsPrefill];
  __shared__ int tb[kMaxExpertsPrefill];
  __shared__ int32_t sid[kRouteThreads];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    run[e] = counts[int64_t(e) * chunks + blockIdx.x];
    tb[e] = tbase[e];
  }
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
      const int pos = run[e] + rank;
      recs[int64_t(tb[e] + pos / kMoeTileRows) * kMoeRecInts + kMoeRecHead + pos % kMoeTileRows] = int32_t(i);
    }
    __syncthreads();  // every thread has read run and sid
    if (ok) atomicAdd(&run[e], 1);
  }
}

// All of the routing in one block (P <= kOneMaxP pairs, E <= kOneMaxE experts), in LDS.
// (1) Per-expert counts (LDS atomics); thread t takes pairs t, t + 1024, ..., kept in
// registers.  (2) Prefixes over the experts of the counts (the buckets' offsets in one flat
// bucket array) and of the tile counts (each expert's first tile); the record heads and
// the table's length are written.  (3) Each pair takes the next free position of its
// expert's bucket (an LDS atomic) and is written there.  (4) The tiles' pair slots are
// copied out, 64 consecutive slots of one record per wave store.  The order inside a
// bucket is whatever order the atomics took, so it may differ from call to call; every
// result is the same, since a pair's outputs are computed with the same operations
// wherever it sits in a tile.
__global__ void __launch_bounds__(kScanThreads) moe_route_one(const int32_t* __restrict__ ids, int P, int E,
                                                              int32_t* __restrict__ hdr,
                                                              int32_t* __restrict__ recs) {
  // The loops below have no branches, so that their LDS operations stay in flight together
  // instead of one round trip each: a lane whose pair has no expert (or is past the end)
  // counts and places it in a spare word of its own (spread over the banks), never read.
  __shared__ int cnt[kOneMaxE + 64];         // pairs per expert, then its next free bucket position
  __shared__ int32_t bucket[kOneMaxP + 64];  // the pairs, bucket after bucket
  __shared__ int tile_off[kOneMaxTiles + 1]; // bucket position of each tile's first pair
  const int tid = threadIdx.x;
  const int spare = kOneMaxE + (tid & 63);
  for (int e = tid; e < kOneMaxE + 64; e += kScanThreads) cnt[e] = 0;
  int32_t v[kOneRegs];  // the pair's expert, or the lane's spare word
#pragma unroll
  for (int k = 0; k < kOneRegs; ++k) {
    const int32_t e = ids[min(tid + k * kScanThreads, P - 1)];
    v[k] = tid + k * kScanThreads < P && routed(e, E) ? e : spare;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOneRegs; ++k) atomicAdd(&cnt[v[k]], 1);  // counts: the order of the adds does not matter
  __syncthreads();
  const int n = tid < E ? cnt[tid] : 0;
  const int t = (n + kMoeTileRows - 1) / kMoeTileRows;
  // both prefixes in one scan: pairs in the low 16 bits, tiles above (n_all <= 16384,
  // t_all < 1152, so neither field carries into the other)
  int packed_all;
  const int packed = block_exclusive_scan(n | (t << 16), &packed_all);
  const int off = packed & 0xFFFF, tb = packed >> 16;
  const int n_all = packed_all & 0xFFFF, t_all = packed_all >> 16;
  if (tid < E) {
    cnt[tid] = off;
    write_heads(recs, tid, n, tb);
    for (int j = 0; j < t; ++j) tile_off[tb + j] = off + j * kMoeTileRows;
  }
  if (tid == 0) {
    tile_off[t_all] = n_all;
    hdr[0] = t_all;
    hdr[1] = n_all;
  }
  __syncthreads();
  // all of a thread's atomics first, then its writes, so that the atomics' round trips overlap
  int pos[kOneRegs];
#pragma unroll
  for (int k = 0; k < kOneRegs; ++k) pos[k] = atomicAdd(&cnt[v[k]], 1);
#pragma unroll
  for (int k = 0; k < kOneRegs; ++k) bucket[v[k] < E ? pos[k] : kOneMaxP + (tid & 63)] = tid + k * kScanThreads;
  __syncthreads();
  // copy-out: 4 slots (16 bytes) per lane and store, kCopyBatch of them per thread at a
  // time (their LDS reads in flight together); a tile ends where the next one starts (the
  // next expert's bucket, for its last tile), and the slots of a partial group past the
  // tile's end take any value (slots past a record's pair count are never read)
  const int quads = t_all * (kMoeTileRows / 4);
  for (int f0 = 0; f0 < quads; f0 += kCopyBatch * kScanThreads) {
    int4 val[kCopyBatch];
    bool ok[kCopyBatch];
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {
      const int f = f0 + k * kScanThreads + tid;
      const int tile = f < quads ? f / (kMoeTileRows / 4) : 0;
      const int lo = tile_off[tile], hi = tile_off[tile + 1];
      const int at = lo + 4 * (f % (kMoeTileRows / 4));
      ok[k] = (f < quads) & (at < hi);
      const int a0 = ok[k] ? at : 0;
      val[k] = make_int4(bucket[a0], bucket[min(a0 + 1, kOneMaxP - 1)], bucket[min(a0 + 2, kOneMaxP - 1)],
                         bucket[min(a0 + 3, kOneMaxP - 1)]);
    }
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {
      const int f = f0 + k * kScanThreads + tid;
      if (ok[k])
        *reinterpret_cast<int4*>(recs + int64_t(f / (kMoeTileRows / 4)) * kMoeRecInts + kMoeRecHead +
                                 4 * (f % (kMoeTileRows / 4))) = val[k];
    }
  }
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
  // every expert's last tile may be partial: fewer than P / 128 + E tiles in all
  L.recs_n = ((L.P + kMoeTileRows - 1) / kMoeTileRows + E + 7) / 8 * 8;
  L.chunk_pairs = route_chunk(L.P);
  L.chunks = (L.P + L.chunk_pairs - 1) / L.chunk_pairs;
  auto up = [](uint64_t b) { return (b + 255) / 256 * 256; };
  uint64_t o = 0;
  L.hdr = o;      o = up(o + 16);
  L.recs = o;     o = up(o + uint64_t(L.recs_n) * kMoeRecInts * 4);
  L.tbase = o;    o = up(o + uint64_t(E) * 4);
  L.chunk = o;    o = up(o + uint64_t(L.chunks) * uint64_t(E) * 4);
  L.z = o;        o = up(o + uint64_t(L.P) * uint64_t(out_rows) * 4);
  L.total = o;
  return L;
}

int launch_moe_route(const int32_t* ids, int64_t M, int64_t topk, int64_t E, void* ws, hipStream_t s) {
  const MoeLayout L = moe_layout(M, topk, E, 0);
  char* b = static_cast<char*>(ws);
  int32_t* hdr = reinterpret_cast<int32_t*>(b + L.hdr);
  int32_t* recs = reinterpret_cast<int32_t*>(b + L.recs);
  if (L.P <= kOneMaxP && E <= kOneMaxE) {
    moe_route_one<<<dim3{1u, 1u, 1u}, dim3{unsigned(kScanThreads), 1u, 1u}, 0, s>>>(ids, int(L.P), int(E), hdr,
                                                                                   recs);
    return hipGetLastError() == hipSuccess ? 0 : 6;
  }
  int32_t* counts = reinterpret_cast<int32_t*>(b + L.chunk);
  int32_t* tbase = reinterpret_cast<int32_t*>(b + L.tbase);
  const dim3 blk{unsigned(kRouteThreads), 1u, 1u};
  const dim3 grid{unsigned(L.chunks), 1u, 1u};
  moe_route_count<<<grid, blk, 0, s>>>(ids, L.P, L.chunk_pairs, int(E), int(L.chunks), counts);
  moe_route_scan<<<dim3{1u, 1u, 1u}, dim3{unsigned(kScanThreads), 1u, 1u}, 0, s>>>(counts, int(L.chunks), int(E),
                                                                                  hdr, tbase, recs);
  moe_route_place<<<grid, blk, 0, s>>>(ids, L.P, L.chunk_pairs, int(E), int(L.chunks), tbase, counts, recs);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int launch_moe_prefill(int stage, const GemmArgs& g, const int32_t* ids, int64_t M, int64_t topk, int64_t E,
                       const void* ws, void* out, hipStream_t s) {
  const MoeLayout L = moe_layout(M, topk, E, stage == 0 ? 0 : g.N);
  const char* b = static_cast<const char*>(ws);
  GemmArgs a = g;
  a.moe_hdr = reinterpret_cast<const int32_t*>(b + L.hdr);
  a.moe_recs = reinterpret_cast<const int32_t*>(b + L.recs);
  if (stage == 0) {
    // stage 1: h [P][I] of the routed pairs from the gathered kernel, whose idle blocks
    // write the zeros of the others
    a.out0 = out;
    a.moe_w = nullptr;
    a.moe_div = topk;
    a.moe_ids = ids;
    a.moe_E = E;
    return launch_moe_gemm(EPI_SWIGLU, a, L.recs_n, s);
  }
  // stage 2: z = p * (D_e h) per routed pair (fp32, workspace), then the per-token sum
  float* z = reinterpret_cast<float*>(const_cast<char*>(b) + L.z);
  const int f32_y = a.f32_out;
  a.out0 = z;
  a.f32_out = 1;
  a.moe_div = 1;
  if (int st = launch_moe_gemm(EPI_LINEAR, a, L.recs_n, s)) return st;
  const unsigned mb = unsigned(M < 4096 ? M : 4096);
  if (a.N % 4 == 0)
    moe_combine<true><<<dim3{mb, 1u, 1u}, dim3{256u, 1u, 1u}, 0, s>>>(ids, M, int(topk), int(E), z, a.N, out, f32_y);
  else
    moe_combine<false><<<dim3{mb, 1u, 1u}, dim3{256u, 1u, 1u}, 0, s>>>(ids, M, int(topk), int(E), z, a.N, out, f32_y);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace qmm
