// Measurement kernels for the roofline legs of the benchmark (not part of the C ABI of
// the quantized matmul): the rate a plain kernel reaches on this GPU for the two
// resources the hot path is bound by.
//   * qmm_ceiling_read: a streaming read of a buffer, no compute, every byte read once
//     with 16-byte loads (one 1 KB piece per wave load instruction, `unroll` pieces in
//     flight per wave), each wave owning either one contiguous slice of the buffer or
//     every (waves)-th group of `unroll` consecutive pieces (interleaved).  Decode is
//     weight-bandwidth bound ("The Cathedral Doubled Itself", what 50 tok/s looks like),
//     so this is the ceiling a GEMV of the same size per launch can approach.
//   * qmm_ceiling_mfma: back-to-back v_mfma_f32_32x32x16_bf16 on registers only (four
//     independent accumulators per wave), the matrix rate the prefill GEMM can approach.
// Built into its own library (libqmm_ceiling.so); only the benchmark loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int U, bool INTERLEAVED>
__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4_t* __restrict__ p, uint64_t pieces,
                                                          uint32_t* __restrict__ sink) {
  const uint64_t lane = threadIdx.x & 63;
  const uint64_t gw = (uint64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const uint64_t nw = (uint64_t(gridDim.x) * blockDim.x) >> 6;
  uint32_t acc = 0;
  if constexpr (INTERLEAVED) {
    // wave gw reads pieces [g*U, g*U + U) for g = gw, gw + nw, ...
    for (uint64_t b = gw * U; b < pieces; b += nw * U) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t i = b + u < pieces ? b + u : pieces - 1;  // clamped: the last group may be short
        v[u] = __builtin_nontemporal_load(p + i * 64 + lane);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][3];
    }
  } else {
    // wave gw reads pieces [b0, b1) of 1 KB (64 lanes x 16 B)
    const uint64_t per = pieces / nw, extra = pieces % nw;
    const uint64_t b0 = gw * per + (gw < extra ? gw : extra);
    const uint64_t b1 = b0 + per + (gw < extra ? 1 : 0);
    uint64_t b = b0;
    for (; b + U <= b1; b += U) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + (b + u) * 64 + lane);
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][3];
    }
    for (; b < b1; ++b) {
      const u32x4_t v = __builtin_nontemporal_load(p + b * 64 + lane);
      acc ^= v[0] ^ v[3];
    }
  }
  // a store that never happens for real data, so the loads are not dead
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __bf16(float((lane + i) & 7) * 0.125f);
    b[i] = __bf16(float((lane * 3 + i) & 7) * 0.0625f);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == -1.2345f) sink[threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 1024, the buffer 16-byte aligned) once; `blocks` blocks of
// 256 threads; `unroll` in {1, 2, 4, 8}; `interleaved` 0 (a contiguous slice per wave) or 1.
// Returns 0, 2 for bad arguments, 6 if the launch failed.  `sink` (256 uint32) is written
// only in a case that real data never produces.
int qmm_ceiling_read(const void* buf, uint64_t bytes, int blocks, int unroll, int interleaved, uint32_t* sink,
                     hipStream_t s) {
  if (!buf || !sink || bytes == 0 || bytes % 1024 || blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15) ||
      (interleaved != 0 && interleaved != 1))
    return 2;
  const u32x4_t* p = static_cast<const u32x4_t*>(buf);
  const uint64_t pieces = bytes / 1024;
#define QMM_CEILING_CASE(U)                                                          \
  case U:                                                                            \
    if (interleaved) read_stream_kernel<U, true><<<blocks, 256, 0, s>>>(p, pieces, sink);  \
    else read_stream_kernel<U, false><<<blocks, 256, 0, s>>>(p, pieces, sink);             \
    break;
  switch (unroll) {
    QMM_CEILING_CASE(1)
    QMM_CEILING_CASE(2)
    QMM_CEILING_CASE(4)
    QMM_CEILING_CASE(8)
    default: return 2;
  }
#undef QMM_CEILING_CASE
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// `blocks` blocks of 4 waves, each wave 4 * iters MFMAs of 32x32x16 (32768 FLOP each).
int qmm_ceiling_mfma(int blocks, int iters, float* sink, hipStream_t s) {
  if (!sink || blocks < 1 || iters < 1) return 2;
  mfma_loop_kernel<<<blocks, 256, 0, s>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
