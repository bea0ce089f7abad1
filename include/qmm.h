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
 *     state (one exception: the scratch array of qmm_moe_prefill_noalloc, below) and
 *     never copies, concatenates or repacks a weight: a fused weight is
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
 *   - M = 1 runs a bandwidth-bound GEMV; M = 2 with K <= 5120 (any format) runs the
 *     same GEMV for both rows against one read of the weights,
 *     each row bit-identical to its own M = 1 call.  For 4-bit group-64 linear / fused
 *     QKV / fused gate+up with K a multiple of 512 up to 8192, otherwise
 *     2 <= M <= 32 (and up to 256 where it
 *     is estimated faster than the GEMM) runs a small-batch kernel that streams the
 *     weights once per 16 or 32 activation rows with the activations on the matrix cores;
 *     otherwise M <= 8 runs the GEMV once per activation row and larger M an
 *     LDS-dequant + MFMA GEMM ("Sanctum-MLX", "Latency testing": prefill is dominated by
 *     the quantized matmuls).  The regimes agree to the tolerance, not bit for bit (the
 *     GEMM rounds dequantized weights to bf16; the reduction orders differ).  Within one
 *     regime a row's result does not depend on the other rows of the call.
 *   - M * K * 2 (the activation bytes) must stay below 4 GiB.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMM_ABI_VERSION 2
#define QMM_MAX_K 65536
#define QMM_MAX_TOPK 64
#define QMM_MAX_EXPERTS_PREFILL 4096
/* size of the library's own device scratch array used by qmm_moe_prefill_noalloc */
#define QMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
/* `bits` of the *_fmt calls for fp8 e4m3 codes (8 bits each) */
#define QMM_FP8_E4M3 0x108

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
 * qmm_fused_qkv_rope -- the fused QKV projection with its split and rotary position
 * embedding in the same kernel: the pages' fused split+RoPE second phase ("Sanctum-MLX",
 * shipped phases table, Phase 2; "The Cathedral Doubled Itself", the kernel that worked
 * and the kernel that won't), which MLX's lazy graph kept from shipping; on a HIP
 * stream the outputs are ordinary stream-ordered results.
 *   Weight rows, in heads of head_dim rows: for each of the n_q_heads query heads its
 *   head_dim query rows and, when q_gate = 1, head_dim output-gate rows right after them
 *   (the doubled q projection of "The Cathedral Doubled Itself", the 35B port); then the
 *   n_kv_heads K heads; then the n_kv_heads V heads.
 *   rows = (n_q_heads * (1 + q_gate) + 2 * n_kv_heads) * head_dim.
 *   Outputs (row-major, separate buffers): q [M][n_q_heads][head_dim],
 *   k and v [M][n_kv_heads][head_dim], gate [M][n_q_heads][head_dim] (q_gate = 1 only;
 *   ignored otherwise).
 *   lin_bias: nullable [rows] bf16, added to each projection before the rotation.
 *   Rotation (Q and K heads; V and gate pass through): for i < rot_dim/2 the dims
 *   (i, i + rot_dim/2) of a head of token m, values (a, b), become
 *   (a*c - b*s, b*c + a*s) with c = cos_sin[p][i], s = cos_sin[p][rot_dim/2 + i],
 *   p = positions[m]; dims [rot_dim, head_dim) pass through.
 *   positions: device int32 [M]; values outside [0, max_pos) are clamped to that range.
 *   cos_sin: device fp32 [max_pos][rot_dim], built once by the caller (cos in the first
 *   half of a row, sin in the second).
 *   head_dim and rot_dim even, 2 <= rot_dim <= head_dim; q_gate 0 or 1.  The regimes are
 *   those of qmm_fused_qkv (the small-batch kernel needs head_dim and rot_dim multiples
 *   of 16 as well).
 */
int qmm_fused_qkv_rope(const uint16_t* x, int64_t M, int64_t K,
                       const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                       int64_t n_q_heads, int64_t n_kv_heads, int64_t head_dim, int q_gate,
                       int64_t rot_dim, const int32_t* positions, const float* cos_sin, int64_t max_pos,
                       const uint16_t* lin_bias, void* q, void* gate, void* k, void* v,
                       int out_dtype, hipStream_t stream);

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

/*
 * qmm_moe_layer -- both stages of qmm_moe_gather for one decode token, in one call (4-bit
 * codes, group 64; the in-place expert grids of "Sanctum-MLX", "Inside the server"):
 *   h = stage QMM_MOE_GATE_UP_SWIGLU of x: gate+up grid gu_* [E][2I][K/8] and [E][2I][K/64],
 *       h [topk][I] bf16, written;
 *   y = stage QMM_MOE_DOWN_COMBINE of h: down grid dn_* [E][K][I/8] and [E][K][I/64],
 *       expert_w fp32 [topk], y [K] in out_dtype.
 * Two launches on `stream` (stage 1, then stage 2, as the two qmm_moe_gather calls); h and
 * y equal those calls' results bit for bit.
 * Shapes: K and I multiples of 64, I <= 5120, topk <= QMM_MAX_TOPK; QMM_ERR_ALIAS if h or y
 * overlap each other or an input.
 */
int qmm_moe_layer(const uint16_t* x, int64_t K, const uint32_t* gu_codes, const uint16_t* gu_scales,
                  const uint16_t* gu_biases, const uint32_t* dn_codes, const uint16_t* dn_scales,
                  const uint16_t* dn_biases, int64_t E, int64_t I, const int32_t* expert_ids, const float* expert_w,
                  int64_t topk, uint16_t* h, void* y, int out_dtype, hipStream_t stream);

/*
 * Routed experts over a batch of tokens (prefill).  Token m has topk (token, slot)
 * pairs p = m*topk + k, each with an expert id expert_ids[m][k] (an id outside [0, E)
 * means "no expert"); the experts are the same in-place 3-D grid as qmm_moe_gather
 * ("Sanctum-MLX", "Inside the server"; never concatenated: "Four Candles for the
 * Cathedral", "What's not in this batch").  Prefill is dominated by the quantized
 * matmuls ("Sanctum-MLX", "Latency testing"), so the pairs are bucketed by expert and
 * each expert's weights are streamed once, through the matrix cores, for all of the
 * tokens routed to it (gathered through the bucket), instead of once per token.
 *
 * Three calls, in stream order:
 *   qmm_moe_route    buckets the pairs of expert_ids by expert into the workspace, as
 *                    records of routing tiles (the order of the pairs inside an
 *                    expert's bucket is not fixed; no result depends on it);
 *   qmm_moe_prefill  stage QMM_MOE_GATE_UP_SWIGLU, then stage QMM_MOE_DOWN_COMBINE,
 *                    both reading that routing.
 * The stages run on a gathered kernel over routing tiles of up to 96 pairs of one expert,
 * each expert row dequantized once per tile.
 * A small batch (M * topk <= 288 pairs: most experts then see one token or none) runs
 * pair by pair instead, on the kernels of qmm_moe_gather: stage 1 one SwiGLU GEMV per
 * (token, slot) pair, stage 2 each token's weighted sum over its slots (expert I <= 5120;
 * a wider one is routed by stage 2 itself and runs the gathered kernel).  The stages then read
 * expert_ids directly and qmm_moe_route does nothing, so the call order above still holds.
 * workspace: caller-owned device memory, 256-byte aligned, of at least
 * qmm_moe_prefill_workspace_bytes(M, topk, E, out_rows) bytes, where out_rows is the
 * row count of the down projection (0 if only stage 1 runs).  It holds the routing
 * (written by qmm_moe_route, read by both stages) and the fp32 per-pair products of
 * stage 2; its contents between calls are the library's.  One workspace serves one
 * routing at a time: calls with different expert_ids on one workspace must be ordered
 * on one stream, route before prefill.  The library still allocates nothing.
 */

/* Workspace bytes for M tokens x topk slots over E experts and a down projection of
 * out_rows rows; 0 when M, topk, E or out_rows is out of range (M in [1, 65535],
 * topk in [1, QMM_MAX_TOPK], E in [1, QMM_MAX_EXPERTS_PREFILL]).  Host only. */
size_t qmm_moe_prefill_workspace_bytes(int64_t M, int64_t topk, int64_t E, int64_t out_rows);

/*
 * qmm_moe_route -- expert_ids: device int32 [M][topk].  Writes the routing into the
 * workspace.  QMM_ERR_SHAPE for sizes out of range or a workspace below
 * qmm_moe_prefill_workspace_bytes(M, topk, E, 0); QMM_ERR_ALIAS if the workspace
 * overlaps expert_ids.
 */
int qmm_moe_route(const int32_t* expert_ids, int64_t M, int64_t topk, int64_t E,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * qmm_moe_prefill -- one stage of the routed experts over M tokens.  expert_ids must be
 * the array (same contents, M, topk, E) the workspace was routed with.
 *   stage QMM_MOE_GATE_UP_SWIGLU: in = x [M][K] bf16; rows = 2*I (gate [0,I), up [I,2I)
 *     of each expert); out h [M][topk][I]: h[m][k] = silu(G_e x_m) * (U_e x_m) for
 *     e = expert_ids[m][k], zero for "no expert".  expert_w is ignored (may be NULL).
 *   stage QMM_MOE_DOWN_COMBINE: in = h [M][topk][K] bf16 (K = I); rows = output size;
 *     expert_w: device fp32 [M][topk]; out y [M][rows] = sum over k = 0..topk-1 of
 *     expert_w[m][k] * (D_e h[m][k]); each product is formed in fp32 and the slots are
 *     added in increasing k (no atomics: deterministic); "no expert" slots add nothing.
 *     The workspace must also hold the fp32 products (out_rows = rows).
 * Like qmm_fused_gate_up_swiglu and qmm_linear in the GEMM regime, the products use
 * bf16-rounded dequantized weights.  Errors as at the top, plus QMM_ERR_SHAPE for a
 * workspace that is too small and QMM_ERR_ALIAS if out or the workspace overlaps an
 * input or each other.
 */
int qmm_moe_prefill(int stage, const uint16_t* in, int64_t M, int64_t K,
                    const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                    int64_t E, int64_t rows, const int32_t* expert_ids, const float* expert_w,
                    int64_t topk, void* workspace, size_t workspace_bytes, void* out, int out_dtype,
                    hipStream_t stream);

/*
 * qmm_moe_prefill_noalloc -- qmm_moe_prefill for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same stage, arguments (without the workspace), kernels and results as
 * qmm_moe_prefill, bit for bit; instead of a caller workspace it uses the library's own
 * file-scope device array of QMM_NOALLOC_SCRATCH_BYTES on the current device (allocated
 * with the library's code on that device and held until the process ends; its device
 * address is looked up on the first call on each device), and each call buckets expert_ids
 * into it itself, so no qmm_moe_route call precedes it.  The call allocates nothing.
 *   Limit: qmm_moe_prefill_workspace_bytes(M, topk, E, stage 1 ? 0 : rows) must not
 *   exceed QMM_NOALLOC_SCRATCH_BYTES (64 MiB: stage 1 of any batch up to 65535 tokens;
 *   stage 2 while pairs * rows * 4 bytes of products fit, e.g. ~4000 (token, slot) pairs
 *   at 2048 output rows); larger sizes return QMM_ERR_SHAPE before anything is enqueued.
 *   Every call on a GPU shares that GPU's one array and leaves its contents behind: two
 *   calls that may run at the same time on one GPU (different streams, or different host
 *   threads without ordering) race on it and give undefined results.  Calls ordered on
 *   one stream are safe.  QMM_ERR_LAUNCH if the array cannot be located on the device.
 */
int qmm_moe_prefill_noalloc(int stage, const uint16_t* in, int64_t M, int64_t K,
                            const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                            int64_t E, int64_t rows, const int32_t* expert_ids, const float* expert_w,
                            int64_t topk, void* out, int out_dtype, hipStream_t stream);

/*
 * A decode step in few launches: several 4-bit group-64 projections of one token (M = 1) run
 * by one launch per dependency level and kind instead of one launch per projection (the
 * pages' case for fusing: 96 launches cost ~3 ms per decode step, "The Cathedral Doubled
 * Itself", "The two fusions"; one command buffer per token, saragossa README, "Design
 * principles").  A projection may read the output of an earlier projection of the same step
 * (the down projection reading its layer's h): it names that projection in wait_for and runs
 * in a later launch of the same run.  Launches: the projections that read no other
 * projection's output form level 0, a projection reading one of level l is of level l + 1;
 * each level is one launch for its projections with K <= 5120 and one for those with a
 * larger K (split over 8 waves; over 16 above K = 40960).  The 14B-shaped step (fused QKV +
 * fused gate+up) is one launch; 40 24B-shaped layers (QKV, gate+up, down) are two.  Nothing
 * waits inside a launch: ordering inside one launch would cost device-scope atomics and
 * cache write-backs per wave, measured at far more than a launch.
 *
 * Every output equals, bit for bit, what the per-call entry point returns for the same
 * projection at M = 1 (qmm_linear, qmm_fused_qkv, qmm_fused_gate_up_swiglu).
 *
 * Two calls:
 *   qmm_step_plan  validates the projections and writes a plan into caller-owned device
 *                  memory of qmm_step_plan_bytes bytes (once, outside graph capture: it
 *                  copies from the host and synchronises `stream`);
 *   qmm_step_run   enqueues a run (its launches, no allocation, no host synchronisation;
 *                  capturable in a HIP graph), as often as needed, with the same
 *                  projections: each run reads the inputs' current contents and
 *                  overwrites the outputs.
 */
enum qmm_step_kind { QMM_STEP_LINEAR = 0, QMM_STEP_QKV = 1, QMM_STEP_GATE_UP_SWIGLU = 2 };

typedef struct qmm_step_proj {
  int32_t kind;            /* QMM_STEP_LINEAR, QMM_STEP_QKV or QMM_STEP_GATE_UP_SWIGLU */
  int32_t wait_for;        /* index of an earlier projection whose output this one's x
                              reads (it then runs in a later launch), or -1 */
  int64_t K;               /* inputs: a multiple of 64, 576 <= K <= QMM_MAX_K */
  int64_t rows;            /* weight rows: N (LINEAR), q_out + 2*kv_out (QKV), 2*I (GATE_UP) */
  int64_t q_out, kv_out;   /* QKV only (ignored otherwise) */
  const uint16_t* x;       /* [K] bf16 */
  const uint32_t* codes;   /* [rows][K/8] */
  const uint16_t* scales;  /* [rows][K/64] bf16 */
  const uint16_t* biases;  /* [rows][K/64] bf16 */
  const uint16_t* lin_bias;  /* nullable [rows] bf16 additive bias; LINEAR and QKV only */
  void* out0;              /* LINEAR: y [rows]; QKV: q [q_out]; GATE_UP: h [rows/2] */
  void* out1;              /* QKV: k [kv_out]; else ignored */
  void* out2;              /* QKV: v [kv_out]; else ignored */
  int32_t out_dtype;       /* QMM_OUT_BF16 or QMM_OUT_F32 */
  int32_t reserved;        /* must be 0 */
} qmm_step_proj;

/* Device bytes of the plan of these n projections (0 if n is outside [1, 4096], or a
 * projection's kind, wait_for or sizes cannot be planned).  Host only; reads kind,
 * wait_for, K, rows. */
size_t qmm_step_plan_bytes(const qmm_step_proj* projs, int32_t n);

/*
 * qmm_step_plan -- projs: host array [n].  plan: device memory, 256-byte aligned, of at
 * least qmm_step_plan_bytes(projs, n) bytes, owned by the caller and left alone between
 * runs.  Checks every projection as the per-call entry points do (QMM_ERR_NULL,
 * QMM_ERR_SHAPE, QMM_ERR_ALIGN, QMM_ERR_ENUM, QMM_ERR_ALIAS), plus: wait_for must be -1 or
 * the index of an earlier projection; outputs may not overlap each other, the plan, or any
 * input, except that a projection's x may lie in the outputs of the projection it waits
 * for.  Then writes the plan (a host-to-device copy on `stream`, followed by
 * hipStreamSynchronize(stream)).  QMM_ERR_LAUNCH if the copy fails.
 */
int qmm_step_plan(const qmm_step_proj* projs, int32_t n, void* plan, size_t plan_bytes, hipStream_t stream);

/*
 * qmm_step_run -- enqueue one run of a plan: projs and n exactly as given to qmm_step_plan
 * for this plan (host, read in full and not checked again: a launch of at most four
 * projections carries them in its kernel arguments, a larger one reads them from the plan).
 * One kernel launch per (level, kind) in order on `stream`; nothing is allocated or copied.
 */
int qmm_step_run(const qmm_step_proj* projs, int32_t n, const void* plan, hipStream_t stream);

/*
 * Other formats of the affine family (saragossa README, "Capabilities": u4/u6/u8 at group
 * sizes 32-128 with bf16 scales/biases; "Quantization formats": u2/u3/u4/u6/u8 affine
 * integer weights).  The *_fmt calls are the calls above with the code width `bits` and
 * the group size `group_size` as their first two arguments; the plain calls are the
 * *_fmt calls at (4, 64).  Layout: codes [rows][K*bits/32] uint32, the row one
 * little-endian bit stream (code k = stream bits [bits*k, bits*k + bits), bit j of the
 * stream = bit j % 32 of word j / 32; at 4 bits this is the nibble order at the top of
 * this file); scales/biases [rows][K/group_size] bf16; w = scale*q + bias, q in
 * 0 .. 2^bits - 1.  bits = QMM_FP8_E4M3: 8-bit codes that are fp8 e4m3 numbers (sign,
 * 4 exponent bits with bias 7, 3 fraction bits, subnormals, S.1111.111 = NaN) and
 * w = scale * e4m3(q) + bias (the pages list fp8 e4m3 with the integer widths without its
 * scaling; this affine form is the reading taken; codes are assumed not NaN).
 * Supported: bits 2, 3, 4, 6, 8, QMM_FP8_E4M3; group_size 32, 64 or 128 with K a
 * multiple of 64 and of group_size; K <= 49152 for 3-, 6- and 8-bit codes (65536
 * otherwise).  Anything else is QMM_ERR_SHAPE.
 */
int qmm_linear_fmt(int bits, int64_t group_size, const uint16_t* x, int64_t M, int64_t K,
                   const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                   int64_t N, const uint16_t* lin_bias, void* y, int out_dtype, hipStream_t stream);
int qmm_fused_qkv_fmt(int bits, int64_t group_size, const uint16_t* x, int64_t M, int64_t K,
                      const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                      int64_t q_out, int64_t kv_out, const uint16_t* lin_bias,
                      void* q, void* k, void* v, int out_dtype, hipStream_t stream);
int qmm_fused_gate_up_swiglu_fmt(int bits, int64_t group_size, const uint16_t* x, int64_t M, int64_t K,
                                 const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                                 int64_t I, void* h, int out_dtype, hipStream_t stream);
int qmm_moe_gather_fmt(int bits, int64_t group_size, int stage, const uint16_t* in, int64_t K,
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
