// Host-side launch interface between the C ABI (qmm_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

// The kernels of each code width (2, 3, 4, 6, 8 bits) are built as their own objects
// from the same sources and live in namespace qmm::b<bits>.
#define QMM_CAT2(a, b) a##b
#define QMM_CAT(a, b) QMM_CAT2(a, b)
#ifndef QMM_FP8
#define QMM_FP8 0
#endif
#if QMM_FP8
#define QMM_BITS_NS f8
#else
#define QMM_BITS_NS QMM_CAT(b, QMM_BITS)
#endif
// Format code of fp8 e4m3 codes in GemvArgs/GemmArgs::bits (QMM_FP8_E4M3 of the C ABI).
constexpr int kFmtFp8E4M3 = 0x108;

enum Epilogue : int { EPI_LINEAR = 0, EPI_QKV = 1, EPI_SWIGLU = 2, EPI_ROPE = 3 };

}  // namespace qmm
struct qmm_step_proj;
namespace qmm {

// Decode step in few launches (gemv_step.hip): plan size (0 if a projection cannot be
// planned), whether a projection's K can be planned, plan writing (validated arguments) and
// the launches of a run.
namespace step {
uint64_t plan_bytes(const qmm_step_proj* projs, int n);
bool shape_ok(const qmm_step_proj& p);
int build_and_upload(const qmm_step_proj* projs, int n, void* plan, uint64_t bytes, hipStream_t stream);
int launch(const qmm_step_proj* projs, int n, const void* plan, hipStream_t stream);
}  // namespace step

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount), queried once
// per device; 256 if the query fails.  The launch geometries are sized from it.
int device_cus();

// Fused QKV with rotary embedding (EPI_ROPE).  The weight is heads of head_dim rows: per
// query head its query rows and, with q_gate, its output-gate rows; then the K heads,
// then the V heads.  Outputs: q -> out0, k -> out1, v -> out2 ([M][heads][head_dim]),
// gate -> `gate`.
struct RopeArgs {
  const int32_t* positions;  // [M] token positions (clamped to [0, max_pos) when read)
  const float* cos_sin;      // [max_pos][rot]: cos in [0, rot/2), sin in [rot/2, rot)
  void* gate;                // [M][n_q][head_dim] output gate (q_gate), else null
  int32_t max_pos, n_q, n_kv, head_dim, rot, q_gate;
};

// Launch geometry of the decode kernels, a function of K only, so a row's
// reduction order never depends on how many rows are in the call (fused and
// unfused projections agree bit for bit).
struct GemvShape {
  int lpr;     // lanes per row slot (16 or 32)
  int cpl;     // 32-code chunks per lane within a K slice
  int ksplit;  // waves sharing one row's K range (their partials meet in LDS)
};

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
  int64_t moe_div;         // stage 1: activation row of slot k is k / moe_div (0: one row)
  int64_t moe_tokens;      // stage 2: tokens, topk slots each (0: one token)
  int topk;                // stage 1: slots (grid.y); stage 2: slots per token
  int f32_out;
  int bits;                // code width (2, 3, 4, 6 or 8) or kFmtFp8E4M3
  int gshift;              // group size = 32 << gshift (scales/biases per 32, 64 or 128 inputs)
  RopeArgs rope;           // EPI_ROPE only
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
  int64_t M, K, N;         // N = weight rows (SWIGLU: 2*I); routed experts: rows of one expert
  int64_t q_out, kv_out, I;
  int f32_out;
  // routed experts over a batch of tokens (gathered GEMM; null otherwise): the tile
  // records written by the routing kernels, and x row = pair / moe_div
  const int32_t* moe_hdr;      // [0] = number of tiles, [1] = routed pairs
  const int32_t* moe_recs;     // [tiles][kMoeRecInts]: expert, pairs n, 0, 0, then n pair indices
  const float* moe_w;          // stage 2: combine weight of each pair; null in stage 1
  int64_t moe_div;             // topk in stage 1 (x row of a pair), 1 in stage 2
  const int32_t* moe_ids;      // stage 1: expert of each pair (the idle blocks zero unrouted h)
  int64_t moe_E;               // stage 1: experts in the grid
  int bits;                    // code width or kFmtFp8E4M3
  int gshift;                  // group size = 32 << gshift
  RopeArgs rope;               // EPI_ROPE only
};

// Launchers of one code width.  Decode GEMV: M rows of x as independent GEMVs (grid.y);
// routed experts for one token: stage 1 (gathered gate+up+SwiGLU), stage 2 (gathered
// down + combine); prefill GEMM (LDS dequant + MFMA).
#define QMM_WIDTH_LAUNCHERS(NS)                                             \
  namespace NS {                                                            \
  bool gemv_shape_for_k(int64_t K, GemvShape* out);                         \
  int launch_gemv(int epi, const GemvArgs& a, int64_t M, hipStream_t s);    \
  int launch_moe_gate_up(const GemvArgs& a, hipStream_t s);                 \
  int launch_moe_down(const GemvArgs& a, hipStream_t s);                    \
  int launch_gemm(int epi, const GemmArgs& a, hipStream_t s);               \
  }
QMM_WIDTH_LAUNCHERS(b2)
QMM_WIDTH_LAUNCHERS(b3)
QMM_WIDTH_LAUNCHERS(b4)
QMM_WIDTH_LAUNCHERS(b6)
QMM_WIDTH_LAUNCHERS(b8)
QMM_WIDTH_LAUNCHERS(f8)
// The routed experts over a batch (4-bit codes, group 64; moe_gemm.hip): each block one
// routing tile x one slab of 128 expert rows (SWIGLU: 64 gate + their 64 up rows);
// m_tiles = the number of tile records (a multiple of 8).
bool moe_gemm_supports(const GemmArgs& a);
int launch_moe_gemm(int epi, const GemmArgs& a, int64_t m_tiles, hipStream_t s);



#define QMM_BY_WIDTH(bits, CALL)                \
  switch (bits) {                               \
    case 2: return b2::CALL;                    \
    case 3: return b3::CALL;                    \
    case 4: return b4::CALL;                    \
    case 6: return b6::CALL;                    \
    case 8: return b8::CALL;                    \
    case kFmtFp8E4M3: return f8::CALL;          \
    default: return 2;                          \
  }
inline int launch_gemv(int epi, const GemvArgs& a, int64_t M, hipStream_t s) {
  QMM_BY_WIDTH(a.bits, launch_gemv(epi, a, M, s))
}
inline int launch_moe_gate_up(const GemvArgs& a, hipStream_t s) { QMM_BY_WIDTH(a.bits, launch_moe_gate_up(a, s)) }
inline int launch_moe_down(const GemvArgs& a, hipStream_t s) { QMM_BY_WIDTH(a.bits, launch_moe_down(a, s)) }
inline int launch_gemm(int epi, const GemmArgs& a, hipStream_t s) { QMM_BY_WIDTH(a.bits, launch_gemm(epi, a, s)) }

// M = 2 on the single-slice decode kernel (K <= 5120, any code width; the rotary
// epilogue for 4-bit codes, like the GEMV itself): both activation rows against one read
// of the weights, each row computed exactly as alone.
#ifndef QMM_GEMV_TWO_ROWS
#define QMM_GEMV_TWO_ROWS 1
#endif
inline bool gemv_two_rows(int64_t K, int64_t M) {
  return QMM_GEMV_TWO_ROWS && M == 2 && K >= 64 && K <= 5120 && K % 64 == 0;
}

// Small batches (2 <= M <= kBmvMaxM) of the 4-bit group-64 projections whose K is a
// multiple of 512 up to 8192: the weights streamed once per 16 or 32 activation rows, the
// activations on the matrix cores (bmv_u4.hip).  Linear, fused QKV, fused gate+up+SwiGLU
// and fused QKV with rotary embedding (head_dim and rot multiples of 16).  bmv_preferred: taken for M <= 32, and above where it beats the
// prefill GEMM's estimate.
constexpr int64_t kBmvMaxM = 256;
bool bmv_supports(int epi, const GemvArgs& a, int64_t M);
bool bmv_preferred(int epi, const GemvArgs& a, int64_t M);
int launch_bmv(int epi, const GemvArgs& a, int64_t M, hipStream_t s);
// Routed experts over a batch (prefill): the workspace holds the bucketed routing and
// the fp32 stage-2 products; all offsets in bytes, 256-byte aligned.
#ifndef QMM_MOE_TILE_ROWS
#define QMM_MOE_TILE_ROWS 96
#endif
constexpr int kMoeTileRows = QMM_MOE_TILE_ROWS;  // pairs per routing tile (a multiple of 32, <= 128)
constexpr int kMaxExpertsPrefill = 4096; // experts the bucketing handles (LDS histogram)
// A routing tile's record: expert, number of pairs n (1 .. kMoeTileRows), two unused words,
// then the tile's pair indices (token * topk + slot) in bucket order; slots past n unused.
constexpr int kMoeRecHead = 4;
constexpr int kMoeRecInts = kMoeRecHead + kMoeTileRows;
struct MoeLayout {
  // pairs, records (a bound on the tiles, rounded up to a multiple of 8), pairs per routing
  // chunk and chunks (the multi-block routing only)
  int64_t P, recs_n, chunk_pairs, chunks;
  uint64_t hdr, recs, tbase, chunk, z, total;
};
MoeLayout moe_layout(int64_t M, int64_t topk, int64_t E, int64_t out_rows);
int launch_moe_route(const int32_t* ids, int64_t M, int64_t topk, int64_t E, void* ws, hipStream_t s);
// stage 0: gate+up+SwiGLU (g.N = 2*I expert rows, out = h [P][I]); stage 1: down + combine
// (g.N = expert rows, out = y [M][N]).  g carries x/h, weights, K, N, I, f32_out.
int launch_moe_prefill(int stage, const GemmArgs& g, const int32_t* ids, int64_t M, int64_t topk, int64_t E,
                       const void* ws, void* out, hipStream_t s);

// qmm_moe_prefill with its checks.  scratch == null: `workspace` is the caller's buffer of
// workspace_bytes, routed by an earlier qmm_moe_route.  scratch != null: workspace is
// ignored; once the sizes are validated against workspace_bytes (the scratch's size),
// scratch(bytes needed) locates the library's own buffer (null: QMM_ERR_LAUNCH), and the
// call buckets expert_ids into it itself before the stage.
int moe_prefill_entry(int stage, const uint16_t* in, int64_t M, int64_t K, const uint32_t* codes,
                      const uint16_t* scales, const uint16_t* biases, int64_t E, int64_t rows,
                      const int32_t* expert_ids, const float* expert_w, int64_t topk, void* workspace,
                      size_t workspace_bytes, void* (*scratch)(size_t), void* out, int out_dtype,
                      hipStream_t stream);


}  // namespace qmm
