/*
 * qmm.h -- C ABI of the MI355X (gfx950) group-wise affine u4 quantized matmul.
 *
 * The operation.  A weight of `rows` output rows over `K` inputs is stored as
 *   codes  [rows][K/8]  uint32: eight 4-bit codes per word along the input axis;
 *                       code k of a row sits at bits 4*(k%8)..4*(k%8)+3 of word
 *                       k/8 (least-significant nibble first);
 *   scales [rows][K/64] bf16 bit patterns, one per 64 consecutive inputs;
 *   biases [rows][K/64] bf16 bit patterns;
 * and stands for w[r][k] = scale[r][k/64] * q[r][k] + bias[r][k/64], q in 0..15.
 * A projection computes y[m][r] = sum_k x[m][k] * w[r][k] with x in bf16.
 *   - 4-bit weights in groups of 64: "Sanctum-MLX" (section "Inside the server":
 *     4-bit QuantizedLinear, group_size=64; model table: 4-bit, group_size=64).
 *   - affine integer weights with bf16 scales and biases, u4 at ~4.5 bits per
 *     weight (= 4 + 2*16/64): saragossa README ("Capabilities"; "Quantization
 *     formats: footprint, throughput & quality").
 *   - eight codes per 32-bit word along the input axis: the fused QKV weight is
 *     [q_out + 2*kv_out, hidden/8] ("2026-05-14: The Cathedral Doubled Itself",
 *     "The two fusions").  The pages do not state the nibble order inside a word;
 *     the least-significant-first order above is this library's reading.
 *
 * Conventions shared by every entry point.
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no pointer after returning, holds no mutable global
 *     state and never copies, concatenates or repacks a weight: a fused weight is
 *     built once by the caller, and the unfused copies can then be dropped
 *     ("2026-05-15: Four Candles for the Cathedral", "#1 -- Drop the fallback
 *     weights").
 *   - Every call takes an explicit stream (0 = the null stream) and returns after
 *     enqueueing; nothing depends on which thread created the stream ("2026-08-17:
 *     The Canary and the Thread-Local Stream", "Thread-local by design").  Inputs
 *     must stay alive and unchanged, and outputs are valid, only once the stream has
 *     reached the work.  A device fault surfaces at the caller's next synchronisation.
 *   - Status: every function returns QMM_OK or an error code and never aborts,
 *     throws or prints.  Arguments are validated before anything is enqueued:
 *       QMM_ERR_NULL   a required pointer is NULL;
 *       QMM_ERR_SHAPE  M < 1, K < 64, K % 64 != 0, K > QMM_MAX_K, a row count < 1,
 *                      topk outside [1, QMM_MAX_TOPK], M > 65535, one weight matrix
 *                      (one expert of a grid) above 4 GiB of codes, or a shape the
 *                      call cannot take;
 *       QMM_ERR_ALIGN  x or codes not 16-byte aligned, a bf16 array not 2-byte
 *                      aligned, an fp32/int32 array or fp32 output not 4-byte aligned;
 *       QMM_ERR_ALIAS  two outputs overlap, or an output overlaps any input (the
 *                      fused outputs are separate contiguous buffers, so the
 *                      view/offset/stride aliasing of "The Cathedral Doubled Itself",
 *                      "The trap that ate three hours", cannot arise);
 *       QMM_ERR_ENUM   unknown out_dtype or MoE stage;
 *       QMM_ERR_LAUNCH the kernel launch failed (hipGetLastError).
 *   - out_dtype: QMM_OUT_BF16 stores bf16 (round to nearest even); QMM_OUT_F32
 *     stores the fp32 value that the bf16 mode would round, so bf16 output ==
 *     RNE(fp32 output) bit for bit.
 *   - Row-major everywhere: x [M][K], y [M][N].  Inputs are assumed finite.
 *   - Decode (M <= 8) runs a bandwidth-bound GEMV, once per activation row; larger M
 *     runs an LDS-dequant + MFMA GEMM ("Sanctum-MLX", "Latency testing": prefill is
 *     dominated by the quantized matmuls).  Results of the two regimes agree to the
 *     tolerance, not bit for bit (the GEMM rounds dequantized weights to bf16).
 *   - M * K * 2 (the activation bytes) must stay below 4 GiB.
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMM_ABI_VERSION 1
#define QMM_MAX_K 65536
#define QMM_MAX_TOPK 64

enum qmm_status {
  QMM_OK = 0,
  QMM_ERR_NULL = 1,
  QMM_ERR_SHAPE = 2,
  QMM_ERR_ALIGN = 3,
  QMM_ERR_ALIAS = 4,
  QMM_ERR_ENUM = 5,
  QMM_ERR_LAUNCH = 6
};

enum qmm_out_dtype { QMM_OUT_BF16 = 0, QMM_OUT_F32 = 1 };

enum qmm_moe_stage { QMM_MOE_GATE_UP_SWIGLU = 0, QMM_MOE_DOWN_COMBINE = 1 };

/*
 * qmm_linear -- one quantized projection: y[m][n] = sum_k x[m][k] * w[n][k]
 * (+ lin_bias[n] when lin_bias != NULL).
 *   x        [M][K] bf16;  codes/scales/biases: N rows over K inputs (see top);
 *   lin_bias nullable [N] bf16;  y [M][N] bf16 or fp32 per out_dtype.
 * The single projection the fusions are built from ("The Cathedral Doubled
 * Itself", "The two fusions"); also the down projection after SwiGLU.
 */
int qmm_linear(const uint16_t* x, int64_t M, int64_t K,
               const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
               const uint16_t* lin_bias, void* y, int out_dtype, hipStream_t stream);

/*
 * qmm_fused_qkv -- one quantized matmul over the row-concatenated q/k/v weight
 * [q_out + 2*kv_out rows][K/8], split into Q, K and V ("2026-05-14: The Cathedral
 * Doubled Itself", "The two fusions", Phase 1A).  Rows [0, q_out) go to q,
 * [q_out, q_out+kv_out) to k, [q_out+kv_out, q_out+2*kv_out) to v; scales and
 * biases are concatenated in the same row order.  q_out is free, so the doubled
 * queries+gate projection ("The Cathedral Doubled Itself", "The 35B port") is the
 * same call.  lin_bias: nullable [q_out + 2*kv_out] bf16 additive output bias.
 *   q [M][q_out], k [M][kv_out], v [M][kv_out]: three separate, non-overlapping,
 *   contiguous row-major buffers ("The trap that ate three hours": each part gets
 *   its own fresh row-major buffer).
 * Each element equals what qmm_linear returns for the same row slice, bit for bit.
 */
int qmm_fused_qkv(const uint16_t* x, int64_t M, int64_t K,
                  const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                  int64_t q_out, int64_t kv_out, const uint16_t* lin_bias,
                  void* q, void* k, void* v, int out_dtype, hipStream_t stream);

/*
 * qmm_fused_gate_up_swiglu -- one quantized matmul over [gate; up] (2*I rows over K
 * inputs: gate rows [0, I), up rows [I, 2I)), then h = silu(gate) * up with
 * silu(g) = g / (1 + exp(-g)), in fp32 ("2026-05-14: The Cathedral Doubled Itself",
 * "The two fusions", Phase 1B: the two parallel matmuls before SiLU+multiply, no
 * additive bias).   h [M][I].
 */
int qmm_fused_gate_up_swiglu(const uint16_t* x, int64_t M, int64_t K,
                             const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                             int64_t I, void* h, int out_dtype, hipStream_t stream);

/*
 * qmm_moe_gather -- routed experts for one decode token, gathered in place from a
 * 3-D expert grid: codes [E][rows][K/8], scales/biases [E][rows][K/64] (the MoE
 * expert grid of "Sanctum-MLX", "Inside the server"; the experts are read where
 * they lie and never concatenated, since concatenated per-expert copies cost ~10 GB
 * and a 6x slowdown: "2026-05-15: Four Candles for the Cathedral", "What's not in
 * this batch").
 *   expert_ids: device int32 [topk]; an id outside [0, E) means "no expert".
 *   stage QMM_MOE_GATE_UP_SWIGLU: in = x [K] bf16; rows = 2*I (gate [0,I), up [I,2I)
 *     of each expert); out [topk][I] = silu(G_e x) * (U_e x) for e = expert_ids[k],
 *     zero for "no expert".  expert_w is ignored (may be NULL).
 *   stage QMM_MOE_DOWN_COMBINE: in = h [topk][K] bf16 (K = I); rows = output size;
 *     expert_w: device fp32 [topk]; out [rows] = sum over k = 0..topk-1
 *     of expert_w[k] * (D_e h[k]), accumulated in fp32 in a fixed order; "no expert"
 *     slots contribute nothing.  No atomics, so the result is deterministic.
 * Ids need not be distinct.  Decode only (one token).  Stage 2 takes K <= 5120.
 */
int qmm_moe_gather(int stage, const uint16_t* in, int64_t K,
                   const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                   int64_t E, int64_t rows, const int32_t* expert_ids, const float* expert_w,
                   int64_t topk, void* out, int out_dtype, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* qmm_status_str(int status);

/* QMM_ABI_VERSION of the built library. */
int qmm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
