// Host-side launch interface between the C ABI (qmm_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qmm {

enum Epilogue : int { EPI_LINEAR = 0, EPI_QKV = 1, EPI_SWIGLU = 2 };

// Launch geometry of the decode kernels, a function of K only, so a row's
// reduction order never depends on how many rows are in the call (fused and
// unfused projections agree bit for bit).
struct GemvShape {
  int lpr;     // lanes per row slot (16 or 32)
  int cpl;     // 32-code chunks per lane within a K slice
  int ksplit;  // waves sharing one row's K range (their partials meet in LDS)
};
bool gemv_shape_for_k(int64_t K, GemvShape* out);

struct GemvArgs {
  const uint16_t* x;       // [M][K] bf16 (stage 2: [topk][K])
  const uint32_t* codes;   // [rows][K/8]            (MoE: expert grid base)
  const uint16_t* scales;  // [rows][K/64]
  const uint16_t* biases;  // [rows][K/64]
  const uint16_t* lin_bias;  // nullable [rows]
  void* out0;              // LINEAR: y; QKV: q; SWIGLU: h; COMBINE: y
  void* out1;              // QKV: k
  void* out2;              // QKV: v
  int64_t K;
  int64_t rows;            // rows of one weight (MoE: rows of one expert)
  int64_t n_out;           // output row stride in elements (M > 1)
  int64_t q_out, kv_out;   // QKV split
  int64_t I;               // SWIGLU: gate rows [0,I), up rows [I,2I)
  const int32_t* expert_ids;  // MoE (nullable otherwise)
  const float* expert_w;      // MoE stage 2
  int64_t E;               // experts in the grid
  int topk;
  int f32_out;
};

struct GemmArgs {
  const uint16_t* x;       // [M][K] bf16
  const uint32_t* codes;   // [N][K/8]
  const uint16_t* scales;  // [N][K/64]
  const uint16_t* biases;  // [N][K/64]
  const uint16_t* lin_bias;  // nullable [N]
  void* out0;              // LINEAR: y [M][N]; QKV: q [M][q_out]; SWIGLU: h [M][I]
  void* out1;              // QKV: k [M][kv_out]
  void* out2;              // QKV: v [M][kv_out]
  int64_t M, K, N;         // N = weight rows (SWIGLU: 2*I)
  int64_t q_out, kv_out, I;
  int f32_out;
};

// Prefill GEMM (LDS dequant + MFMA).
int launch_gemm(int epi, const GemmArgs& a, hipStream_t s);

// Decode GEMV; M rows of x processed as independent GEMVs (grid.y).
int launch_gemv(int epi, const GemvArgs& a, int64_t M, hipStream_t s);
// Routed experts: stage 1 (gathered gate+up+SwiGLU) and stage 2 (gathered down + combine).
int launch_moe_gate_up(const GemvArgs& a, hipStream_t s);
int launch_moe_down(const GemvArgs& a, hipStream_t s);

}  // namespace qmm
