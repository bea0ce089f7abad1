// C ABI entry points (declared and documented in include/qmm.h): validate, then
// enqueue the kernel for the regime (decode GEMV, small-batch MFMA kernel, LDS-dequant +
// MFMA GEMM; see include/qmm.h).  Nothing here allocates, synchronises or keeps state.
#include <hip/hip_runtime_api.h>

#include <atomic>

#include "qmm.h"
#include "qmm_internal.h"
#include "qmm_validate.h"

using qmm::Range;

namespace qmm {
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess || cus < 1)
    cus = 256;
  if (dev >= 0) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}
}  // namespace qmm

static_assert(QMM_MAX_EXPERTS_PREFILL == qmm::kMaxExpertsPrefill, "routing histogram size");
static_assert(QMM_FP8_E4M3 == qmm::kFmtFp8E4M3, "fp8 format code");

namespace {

bool out_dtype_ok(int d) { return d == QMM_OUT_BF16 || d == QMM_OUT_F32; }

// The kernels address the activations with 32-bit byte offsets.
bool acts_fit(int64_t M, int64_t K) { return uint64_t(M) * uint64_t(K) * 2 <= 0xFFFFFFFFull; }

// Activation rows up to which the decode GEMV runs (once per row); above, the GEMM.
constexpr int64_t kGemvMaxM = 8;
#ifndef QMM_MOE_PAIRS_BY_GEMV
#define QMM_MOE_PAIRS_BY_GEMV 288
#endif
// Routed experts over a batch: up to this many (token, slot) pairs run pair by pair
// (measured on the 35B-A3B shape, route included: at 32 tokens x top-8 the layer takes
// 110 us pair by pair against 119 us through the routed path, at 40 tokens 139 against
// 123 us; the pair path grows ~0.39 us per pair, the routed one ~0.1 us).
constexpr int64_t kMoePairsByGemv = QMM_MOE_PAIRS_BY_GEMV;

// A format of the affine family: code width and group size (the pages list u2 .. u8 at
// group sizes 32 to 128: saragossa README, "Capabilities" and "Quantization formats").
struct Fmt {
  int bits;        // format code passed to the kernels: 2, 3, 4, 6, 8 or QMM_FP8_E4M3
  int gshift;      // group = 32 << gshift
  int64_t group;
  int storage;     // bits per code in memory
};
// The widths the kernels implement; false for others, for other group sizes, and when K
// is not a whole number of groups.
bool fmt_ok(int bits, int64_t group, int64_t K, Fmt* f) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 6 && bits != 8 && bits != QMM_FP8_E4M3) return false;
  const int storage = bits == QMM_FP8_E4M3 ? 8 : bits;
  int gs;
  if (group == 32) gs = 0;
  else if (group == 64) gs = 1;
  else if (group == 128) gs = 2;
  else return false;
  if (K % group) return false;
  // the widest codes fit the decode kernel's 16-way K split up to K = 16 * 32 * 3 * 32
  if ((storage == 3 || storage == 6 || storage == 8) && K > 49152) return false;
  *f = {bits, gs, group, storage};
  return true;
}
constexpr Fmt kU4G64 = {4, 1, 64, 4};
uint64_t code_bytes(int64_t rows, int64_t K, const Fmt& f) { return uint64_t(rows) * uint64_t(K) * f.storage / 8; }
uint64_t group_bytes(int64_t rows, int64_t K, const Fmt& f) { return uint64_t(rows) * uint64_t(K / f.group) * 2; }
// One weight matrix (one expert of a grid) is addressed with 32-bit byte offsets.
bool codes_fit(int64_t rows, int64_t K, const Fmt& f) { return code_bytes(rows, K, f) <= 0xFFFFFFFFull; }

qmm::GemmArgs gemm_args(const qmm::GemvArgs& g, int64_t M, int64_t N) {
  qmm::GemmArgs a = {};
  a.x = g.x;
  a.codes = g.codes;
  a.scales = g.scales;
  a.biases = g.biases;
  a.lin_bias = g.lin_bias;
  a.out0 = g.out0;
  a.out1 = g.out1;
  a.out2 = g.out2;
  a.M = M;
  a.K = g.K;
  a.N = N;
  a.q_out = g.q_out;
  a.kv_out = g.kv_out;
  a.I = g.I;
  a.f32_out = g.f32_out;
  a.bits = g.bits;
  a.gshift = g.gshift;
  a.rope = g.rope;
  return a;
}
size_t out_elem(int d) { return d == QMM_OUT_F32 ? 4 : 2; }

int check_weight(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases) {
  if (!x || !codes || !scales || !biases) return QMM_ERR_NULL;
  if (!qmm::aligned(x, 16) || !qmm::aligned(codes, 16) || !qmm::aligned(scales, 2) || !qmm::aligned(biases, 2))
    return QMM_ERR_ALIGN;
  return QMM_OK;
}

}  // namespace

extern "C" {

int qmm_abi_version(void) { return QMM_ABI_VERSION; }

const char* qmm_status_str(int status) {
  switch (status) {
    case QMM_OK: return "QMM_OK";
    case QMM_ERR_NULL: return "QMM_ERR_NULL: a required pointer is NULL";
    case QMM_ERR_SHAPE: return "QMM_ERR_SHAPE: unsupported or inconsistent sizes";
    case QMM_ERR_ALIGN: return "QMM_ERR_ALIGN: misaligned pointer";
    case QMM_ERR_ALIAS: return "QMM_ERR_ALIAS: an output overlaps another output or an input";
    case QMM_ERR_ENUM: return "QMM_ERR_ENUM: unknown out_dtype or stage";
    case QMM_ERR_LAUNCH: return "QMM_ERR_LAUNCH: kernel launch failed";
    default: return "QMM_ERR_UNKNOWN";
  }
}

int qmm_linear_fmt(int bits, int64_t group_size, const uint16_t* x, int64_t M, int64_t K, const uint32_t* codes,
                   const uint16_t* scales, const uint16_t* biases, int64_t N, const uint16_t* lin_bias, void* y,
                   int out_dtype, hipStream_t stream) {
  if (int st = check_weight(x, codes, scales, biases)) return st;
  if (!y) return QMM_ERR_NULL;
  if (!out_dtype_ok(out_dtype)) return QMM_ERR_ENUM;
  Fmt f;
  if (M < 1 || N < 1 || !qmm::k_ok(K) || M > 65535 || !fmt_ok(bits, group_size, K, &f) || !codes_fit(N, K, f) ||
      !acts_fit(M, K))
    return QMM_ERR_SHAPE;
  if (!qmm::aligned(y, out_elem(out_dtype)) || (lin_bias && !qmm::aligned(lin_bias, 2))) return QMM_ERR_ALIGN;
  const Range outs[] = {{y, uint64_t(M * N) * out_elem(out_dtype)}};
  const Range ins[] = {{x, uint64_t(M * K) * 2},
                       {codes, code_bytes(N, K, f)},
                       {scales, group_bytes(N, K, f)},
                       {biases, group_bytes(N, K, f)},
                       {lin_bias, lin_bias ? uint64_t(N) * 2 : 0}};
  if (qmm::any_alias(outs, 1, ins, 5)) return QMM_ERR_ALIAS;

  qmm::GemvArgs a = {};
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.lin_bias = lin_bias;
  a.out0 = y;
  a.K = K;
  a.rows = N;
  a.n_out = N;
  a.f32_out = out_dtype == QMM_OUT_F32;
  a.bits = f.bits;
  a.gshift = f.gshift;
  if (qmm::bmv_preferred(qmm::EPI_LINEAR, a, M)) return qmm::launch_bmv(qmm::EPI_LINEAR, a, M, stream);
  if (M > kGemvMaxM) return qmm::launch_gemm(qmm::EPI_LINEAR, gemm_args(a, M, N), stream);
  return qmm::launch_gemv(qmm::EPI_LINEAR, a, M, stream);
}

int qmm_linear(const uint16_t* x, int64_t M, int64_t K, const uint32_t* codes, const uint16_t* scales,
               const uint16_t* biases, int64_t N, const uint16_t* lin_bias, void* y, int out_dtype,
               hipStream_t stream) {
  return qmm_linear_fmt(kU4G64.bits, kU4G64.group, x, M, K, codes, scales, biases, N, lin_bias, y, out_dtype,
                        stream);
}

int qmm_fused_qkv_fmt(int bits, int64_t group_size, const uint16_t* x, int64_t M, int64_t K, const uint32_t* codes,
                      const uint16_t* scales, const uint16_t* biases, int64_t q_out, int64_t kv_out,
                      const uint16_t* lin_bias, void* q, void* k, void* v, int out_dtype, hipStream_t stream) {
  if (int st = check_weight(x, codes, scales, biases)) return st;
  if (!q || !k || !v) return QMM_ERR_NULL;
  if (!out_dtype_ok(out_dtype)) return QMM_ERR_ENUM;
  const int64_t rows = q_out + 2 * kv_out;
  Fmt f;
  if (M < 1 || q_out < 1 || kv_out < 1 || !qmm::k_ok(K) || M > 65535 || !fmt_ok(bits, group_size, K, &f) ||
      !codes_fit(rows, K, f) || !acts_fit(M, K))
    return QMM_ERR_SHAPE;
  const size_t e = out_elem(out_dtype);
  if (!qmm::aligned(q, e) || !qmm::aligned(k, e) || !qmm::aligned(v, e) || (lin_bias && !qmm::aligned(lin_bias, 2)))
    return QMM_ERR_ALIGN;
  const Range outs[] = {{q, uint64_t(M * q_out) * e}, {k, uint64_t(M * kv_out) * e}, {v, uint64_t(M * kv_out) * e}};
  const Range ins[] = {{x, uint64_t(M * K) * 2},
                       {codes, code_bytes(rows, K, f)},
                       {scales, group_bytes(rows, K, f)},
                       {biases, group_bytes(rows, K, f)},
                       {lin_bias, lin_bias ? uint64_t(rows) * 2 : 0}};
  if (qmm::any_alias(outs, 3, ins, 5)) return QMM_ERR_ALIAS;

  qmm::GemvArgs a = {};
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.lin_bias = lin_bias;
  a.out0 = q;
  a.out1 = k;
  a.out2 = v;
  a.K = K;
  a.rows = rows;
  a.q_out = q_out;
  a.kv_out = kv_out;
  a.f32_out = out_dtype == QMM_OUT_F32;
  a.bits = f.bits;
  a.gshift = f.gshift;
  if (qmm::bmv_preferred(qmm::EPI_QKV, a, M)) return qmm::launch_bmv(qmm::EPI_QKV, a, M, stream);
  if (M > kGemvMaxM) return qmm::launch_gemm(qmm::EPI_QKV, gemm_args(a, M, rows), stream);
  return qmm::launch_gemv(qmm::EPI_QKV, a, M, stream);
}

int qmm_fused_qkv(const uint16_t* x, int64_t M, int64_t K, const uint32_t* codes, const uint16_t* scales,
                  const uint16_t* biases, int64_t q_out, int64_t kv_out, const uint16_t* lin_bias, void* q, void* k,
                  void* v, int out_dtype, hipStream_t stream) {
  return qmm_fused_qkv_fmt(kU4G64.bits, kU4G64.group, x, M, K, codes, scales, biases, q_out, kv_out, lin_bias, q, k,
                           v, out_dtype, stream);
}

int qmm_fused_qkv_rope(const uint16_t* x, int64_t M, int64_t K, const uint32_t* codes, const uint16_t* scales,
                       const uint16_t* biases, int64_t n_q_heads, int64_t n_kv_heads, int64_t head_dim, int q_gate,
                       int64_t rot_dim, const int32_t* positions, const float* cos_sin, int64_t max_pos,
                       const uint16_t* lin_bias, void* q, void* gate, void* k, void* v, int out_dtype,
                       hipStream_t stream) {
  if (int st = check_weight(x, codes, scales, biases)) return st;
  if (!q || !k || !v || !positions || !cos_sin || (q_gate && !gate)) return QMM_ERR_NULL;
  if (!out_dtype_ok(out_dtype)) return QMM_ERR_ENUM;
  const int64_t lim = int64_t(1) << 20;
  if (M < 1 || M > 65535 || !qmm::k_ok(K) || n_q_heads < 1 || n_q_heads > lim || n_kv_heads < 1 ||
      n_kv_heads > lim || head_dim < 2 || head_dim % 2 || head_dim > lim || (q_gate != 0 && q_gate != 1) ||
      rot_dim < 2 || rot_dim % 2 || rot_dim > head_dim || max_pos < 1 || max_pos > (int64_t(1) << 31) - 1)
    return QMM_ERR_SHAPE;
  const int64_t rows = (n_q_heads * (1 + q_gate) + 2 * n_kv_heads) * head_dim;
  if (rows > (int64_t(1) << 30) || !codes_fit(rows, K, kU4G64) || !acts_fit(M, K) ||
      uint64_t(max_pos) * uint64_t(rot_dim) > (uint64_t(1) << 40))
    return QMM_ERR_SHAPE;
  const size_t e = out_elem(out_dtype);
  if (!qmm::aligned(q, e) || !qmm::aligned(k, e) || !qmm::aligned(v, e) || (q_gate && !qmm::aligned(gate, e)) ||
      !qmm::aligned(positions, 4) || !qmm::aligned(cos_sin, 4) || (lin_bias && !qmm::aligned(lin_bias, 2)))
    return QMM_ERR_ALIGN;
  const uint64_t qn = uint64_t(M * n_q_heads * head_dim) * e, kvn = uint64_t(M * n_kv_heads * head_dim) * e;
  const Range outs[] = {{q, qn}, {k, kvn}, {v, kvn}, {q_gate ? gate : nullptr, q_gate ? qn : 0}};
  const Range ins[] = {{x, uint64_t(M * K) * 2},
                       {codes, code_bytes(rows, K, kU4G64)},
                       {scales, group_bytes(rows, K, kU4G64)},
                       {biases, group_bytes(rows, K, kU4G64)},
                       {lin_bias, lin_bias ? uint64_t(rows) * 2 : 0},
                       {positions, uint64_t(M) * 4},
                       {cos_sin, uint64_t(max_pos) * uint64_t(rot_dim) * 4}};
  if (qmm::any_alias(outs, 4, ins, 7)) return QMM_ERR_ALIAS;

  qmm::GemvArgs a = {};
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.lin_bias = lin_bias;
  a.out0 = q;
  a.out1 = k;
  a.out2 = v;
  a.K = K;
  a.rows = rows;
  a.f32_out = out_dtype == QMM_OUT_F32;
  a.bits = 4;
  a.gshift = kU4G64.gshift;
  a.rope.positions = positions;
  a.rope.cos_sin = cos_sin;
  a.rope.gate = q_gate ? gate : nullptr;
  a.rope.max_pos = int32_t(max_pos);
  a.rope.n_q = int32_t(n_q_heads);
  a.rope.n_kv = int32_t(n_kv_heads);
  a.rope.head_dim = int32_t(head_dim);
  a.rope.rot = int32_t(rot_dim);
  a.rope.q_gate = q_gate;
  if (qmm::bmv_preferred(qmm::EPI_ROPE, a, M)) return qmm::launch_bmv(qmm::EPI_ROPE, a, M, stream);
  if (M > kGemvMaxM) return qmm::launch_gemm(qmm::EPI_ROPE, gemm_args(a, M, rows), stream);
  return qmm::launch_gemv(qmm::EPI_ROPE, a, M, stream);
}

int qmm_fused_gate_up_swiglu_fmt(int bits, int64_t group_size, const uint16_t* x, int64_t M, int64_t K,
                                 const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t I,
                                 void* h, int out_dtype, hipStream_t stream) {
  if (int st = check_weight(x, codes, scales, biases)) return st;
  if (!h) return QMM_ERR_NULL;
  if (!out_dtype_ok(out_dtype)) return QMM_ERR_ENUM;
  Fmt f;
  if (M < 1 || I < 1 || !qmm::k_ok(K) || M > 65535 || !fmt_ok(bits, group_size, K, &f) || !codes_fit(2 * I, K, f) ||
      !acts_fit(M, K))
    return QMM_ERR_SHAPE;
  if (!qmm::aligned(h, out_elem(out_dtype))) return QMM_ERR_ALIGN;
  const Range outs[] = {{h, uint64_t(M * I) * out_elem(out_dtype)}};
  const Range ins[] = {{x, uint64_t(M * K) * 2},
                       {codes, code_bytes(2 * I, K, f)},
                       {scales, group_bytes(2 * I, K, f)},
                       {biases, group_bytes(2 * I, K, f)}};
  if (qmm::any_alias(outs, 1, ins, 4)) return QMM_ERR_ALIAS;

  qmm::GemvArgs a = {};
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.out0 = h;
  a.K = K;
  a.rows = 2 * I;
  a.I = I;
  a.n_out = I;
  a.f32_out = out_dtype == QMM_OUT_F32;
  a.bits = f.bits;
  a.gshift = f.gshift;
  if (qmm::bmv_preferred(qmm::EPI_SWIGLU, a, M)) return qmm::launch_bmv(qmm::EPI_SWIGLU, a, M, stream);
  if (M > kGemvMaxM) return qmm::launch_gemm(qmm::EPI_SWIGLU, gemm_args(a, M, 2 * I), stream);
  return qmm::launch_gemv(qmm::EPI_SWIGLU, a, M, stream);
}

int qmm_fused_gate_up_swiglu(const uint16_t* x, int64_t M, int64_t K, const uint32_t* codes,
                             const uint16_t* scales, const uint16_t* biases, int64_t I, void* h, int out_dtype,
                             hipStream_t stream) {
  return qmm_fused_gate_up_swiglu_fmt(kU4G64.bits, kU4G64.group, x, M, K, codes, scales, biases, I, h, out_dtype,
                                      stream);
}

int qmm_moe_gather_fmt(int bits, int64_t group_size, int stage, const uint16_t* in, int64_t K,
                       const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t E, int64_t rows,
                       const int32_t* expert_ids, const float* expert_w, int64_t topk, void* out, int out_dtype,
                       hipStream_t stream) {
  if (stage != QMM_MOE_GATE_UP_SWIGLU && stage != QMM_MOE_DOWN_COMBINE) return QMM_ERR_ENUM;
  if (int st = check_weight(in, codes, scales, biases)) return st;
  if (!expert_ids || !out || (stage == QMM_MOE_DOWN_COMBINE && !expert_w)) return QMM_ERR_NULL;
  if (!out_dtype_ok(out_dtype)) return QMM_ERR_ENUM;
  Fmt f;
  if (!qmm::k_ok(K) || E < 1 || rows < 1 || topk < 1 || topk > QMM_MAX_TOPK || E > (int64_t(1) << 24) ||
      !fmt_ok(bits, group_size, K, &f) || !codes_fit(rows, K, f))
    return QMM_ERR_SHAPE;
  if (stage == QMM_MOE_GATE_UP_SWIGLU && rows % 2) return QMM_ERR_SHAPE;
  if (stage == QMM_MOE_DOWN_COMBINE && K > 5120) return QMM_ERR_SHAPE;
  const size_t e = out_elem(out_dtype);
  if (!qmm::aligned(out, e) || !qmm::aligned(expert_ids, 4) || (expert_w && !qmm::aligned(expert_w, 4)))
    return QMM_ERR_ALIGN;
  const int64_t in_elems = stage == QMM_MOE_GATE_UP_SWIGLU ? K : topk * K;
  const int64_t out_elems = stage == QMM_MOE_GATE_UP_SWIGLU ? topk * (rows / 2) : rows;
  const Range outs[] = {{out, uint64_t(out_elems) * e}};
  const Range ins[] = {{in, uint64_t(in_elems) * 2},
                       {codes, code_bytes(E * rows, K, f)},
                       {scales, group_bytes(E * rows, K, f)},
                       {biases, group_bytes(E * rows, K, f)},
                       {expert_ids, uint64_t(topk) * 4},
                       {expert_w, expert_w ? uint64_t(topk) * 4 : 0}};
  if (qmm::any_alias(outs, 1, ins, 6)) return QMM_ERR_ALIAS;

  qmm::GemvArgs a = {};
  a.x = in;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.out0 = out;
  a.K = K;
  a.rows = rows;
  a.I = rows / 2;
  a.expert_ids = expert_ids;
  a.expert_w = expert_w;
  a.E = E;
  a.topk = int(topk);
  a.f32_out = out_dtype == QMM_OUT_F32;
  a.bits = f.bits;
  a.gshift = f.gshift;
  if (stage == QMM_MOE_GATE_UP_SWIGLU) return qmm::launch_moe_gate_up(a, stream);
  return qmm::launch_moe_down(a, stream);
}

int qmm_moe_gather(int stage, const uint16_t* in, int64_t K, const uint32_t* codes, const uint16_t* scales,
                   const uint16_t* biases, int64_t E, int64_t rows, const int32_t* expert_ids,
                   const float* expert_w, int64_t topk, void* out, int out_dtype, hipStream_t stream) {
  return qmm_moe_gather_fmt(kU4G64.bits, kU4G64.group, stage, in, K, codes, scales, biases, E, rows, expert_ids,
                            expert_w, topk, out, out_dtype, stream);
}

int qmm_moe_layer(const uint16_t* x, int64_t K, const uint32_t* gu_codes, const uint16_t* gu_scales,
                  const uint16_t* gu_biases, const uint32_t* dn_codes, const uint16_t* dn_scales,
                  const uint16_t* dn_biases, int64_t E, int64_t I, const int32_t* expert_ids, const float* expert_w,
                  int64_t topk, uint16_t* h, void* y, int out_dtype, hipStream_t stream) {
  if (int st = check_weight(x, gu_codes, gu_scales, gu_biases)) return st;
  if (!dn_codes || !dn_scales || !dn_biases || !expert_ids || !expert_w || !h || !y) return QMM_ERR_NULL;
  if (!out_dtype_ok(out_dtype)) return QMM_ERR_ENUM;
  const Fmt& f = kU4G64;
  if (!qmm::k_ok(K) || !qmm::k_ok(I) || I > 5120 || E < 1 || E > (int64_t(1) << 24) || topk < 1 ||
      topk > QMM_MAX_TOPK || !codes_fit(2 * I, K, f) || !codes_fit(K, I, f))
    return QMM_ERR_SHAPE;
  const size_t e = out_elem(out_dtype);
  if (!qmm::aligned(dn_codes, 16) || !qmm::aligned(dn_scales, 2) || !qmm::aligned(dn_biases, 2) ||
      !qmm::aligned(h, 16) || !qmm::aligned(y, e) || !qmm::aligned(expert_ids, 4) || !qmm::aligned(expert_w, 4))
    return QMM_ERR_ALIGN;
  const Range outs[] = {{h, uint64_t(topk * I) * 2}, {y, uint64_t(K) * e}};
  const Range ins[] = {{x, uint64_t(K) * 2},
                       {gu_codes, code_bytes(E * 2 * I, K, f)},
                       {gu_scales, group_bytes(E * 2 * I, K, f)},
                       {gu_biases, group_bytes(E * 2 * I, K, f)},
                       {dn_codes, code_bytes(E * K, I, f)},
                       {dn_scales, group_bytes(E * K, I, f)},
                       {dn_biases, group_bytes(E * K, I, f)},
                       {expert_ids, uint64_t(topk) * 4},
                       {expert_w, uint64_t(topk) * 4}};
  if (qmm::any_alias(outs, 2, ins, 9)) return QMM_ERR_ALIAS;

  // the two stages exactly as qmm_moe_gather takes them
  qmm::GemvArgs a1 = {};
  a1.x = x;
  a1.codes = gu_codes;
  a1.scales = gu_scales;
  a1.biases = gu_biases;
  a1.out0 = h;
  a1.K = K;
  a1.rows = 2 * I;
  a1.I = I;
  a1.expert_ids = expert_ids;
  a1.E = E;
  a1.topk = int(topk);
  a1.bits = f.bits;
  a1.gshift = f.gshift;
  qmm::GemvArgs a2 = {};
  a2.x = h;
  a2.codes = dn_codes;
  a2.scales = dn_scales;
  a2.biases = dn_biases;
  a2.out0 = y;
  a2.K = I;
  a2.rows = K;
  a2.I = K / 2;
  a2.expert_ids = expert_ids;
  a2.expert_w = expert_w;
  a2.E = E;
  a2.topk = int(topk);
  a2.f32_out = out_dtype == QMM_OUT_F32;
  a2.bits = f.bits;
  a2.gshift = f.gshift;
  if (int st = qmm::launch_moe_gate_up(a1, stream)) return st;
  return qmm::launch_moe_down(a2, stream);
}

size_t qmm_moe_prefill_workspace_bytes(int64_t M, int64_t topk, int64_t E, int64_t out_rows) {
  if (M < 1 || M > 65535 || topk < 1 || topk > QMM_MAX_TOPK || E < 1 || E > QMM_MAX_EXPERTS_PREFILL ||
      out_rows < 0 || out_rows > (int64_t(1) << 24))
    return 0;
  return size_t(qmm::moe_layout(M, topk, E, out_rows).total);
}

int qmm_moe_route(const int32_t* expert_ids, int64_t M, int64_t topk, int64_t E, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  if (!expert_ids || !workspace) return QMM_ERR_NULL;
  const size_t need = qmm_moe_prefill_workspace_bytes(M, topk, E, 0);
  if (need == 0 || workspace_bytes < need) return QMM_ERR_SHAPE;
  if (!qmm::aligned(expert_ids, 4) || !qmm::aligned(workspace, 256)) return QMM_ERR_ALIGN;
  const Range outs[] = {{workspace, uint64_t(need)}};
  const Range ins[] = {{expert_ids, uint64_t(M * topk) * 4}};
  if (qmm::any_alias(outs, 1, ins, 1)) return QMM_ERR_ALIAS;
  // a small batch runs pair by pair and reads expert_ids directly: nothing to bucket
  if (M * topk <= kMoePairsByGemv) return QMM_OK;
  return qmm::launch_moe_route(expert_ids, M, topk, E, workspace, stream);
}

// ---- decode step in one launch -----------------------------------------------------------

namespace {

constexpr int32_t kMaxStepProjections = 4096;

// Per-projection checks of qmm_step_plan, in the order of the per-call entry points.
int check_step_proj(const qmm_step_proj& p, int32_t index) {
  if (p.kind != QMM_STEP_LINEAR && p.kind != QMM_STEP_QKV && p.kind != QMM_STEP_GATE_UP_SWIGLU) return QMM_ERR_ENUM;
  if (int st = check_weight(p.x, p.codes, p.scales, p.biases)) return st;
  if (!p.out0 || (p.kind == QMM_STEP_QKV && (!p.out1 || !p.out2))) return QMM_ERR_NULL;
  if (!out_dtype_ok(p.out_dtype)) return QMM_ERR_ENUM;
  if (p.reserved != 0 || p.wait_for < -1 || p.wait_for >= index || !qmm::k_ok(p.K) || p.K <= 512 ||
      p.rows < 1 || p.rows > (int64_t(1) << 30) || !codes_fit(p.rows, p.K, kU4G64))
    return QMM_ERR_SHAPE;
  if (p.kind == QMM_STEP_QKV && (p.q_out < 1 || p.kv_out < 1 || p.q_out + 2 * p.kv_out != p.rows))
    return QMM_ERR_SHAPE;
  if (p.kind == QMM_STEP_GATE_UP_SWIGLU && (p.rows % 2 || p.lin_bias)) return QMM_ERR_SHAPE;
  if (!qmm::step::shape_ok(p)) return QMM_ERR_SHAPE;
  const size_t e = out_elem(p.out_dtype);
  if (!qmm::aligned(p.out0, e) || (p.kind == QMM_STEP_QKV && (!qmm::aligned(p.out1, e) || !qmm::aligned(p.out2, e))) ||
      (p.lin_bias && !qmm::aligned(p.lin_bias, 2)))
    return QMM_ERR_ALIGN;
  return QMM_OK;
}

// The output ranges of a projection (1 or 3).
int step_outputs(const qmm_step_proj& p, Range* r) {
  const uint64_t e = out_elem(p.out_dtype);
  if (p.kind == QMM_STEP_QKV) {
    r[0] = {p.out0, uint64_t(p.q_out) * e};
    r[1] = {p.out1, uint64_t(p.kv_out) * e};
    r[2] = {p.out2, uint64_t(p.kv_out) * e};
    return 3;
  }
  r[0] = {p.out0, uint64_t(p.kind == QMM_STEP_GATE_UP_SWIGLU ? p.rows / 2 : p.rows) * e};
  return 1;
}

// The input ranges of a projection (x first).
int step_inputs(const qmm_step_proj& p, Range* r) {
  r[0] = {p.x, uint64_t(p.K) * 2};
  r[1] = {p.codes, code_bytes(p.rows, p.K, kU4G64)};
  r[2] = {p.scales, group_bytes(p.rows, p.K, kU4G64)};
  r[3] = {p.biases, group_bytes(p.rows, p.K, kU4G64)};
  r[4] = {p.lin_bias, p.lin_bias ? uint64_t(p.rows) * 2 : 0};
  return 5;
}

bool overlap(const Range& a, const Range& b) {
  return qmm::any_alias(&a, 1, &b, 1);
}

}  // namespace

size_t qmm_step_plan_bytes(const qmm_step_proj* projs, int32_t n) {
  if (!projs || n < 1 || n > kMaxStepProjections) return 0;
  for (int32_t i = 0; i < n; ++i) {
    const qmm_step_proj& p = projs[i];
    if ((p.kind != QMM_STEP_LINEAR && p.kind != QMM_STEP_QKV && p.kind != QMM_STEP_GATE_UP_SWIGLU) ||
        p.wait_for < -1 || p.wait_for >= i || !qmm::k_ok(p.K) || p.K <= 512 || p.rows < 1 ||
        p.rows > (int64_t(1) << 30))
      return 0;
  }
  return size_t(qmm::step::plan_bytes(projs, n));
}

int qmm_step_plan(const qmm_step_proj* projs, int32_t n, void* plan, size_t plan_bytes, hipStream_t stream) {
  if (!projs || !plan) return QMM_ERR_NULL;
  if (n < 1 || n > kMaxStepProjections) return QMM_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (int st = check_step_proj(projs[i], i)) return st;
  const size_t need = qmm_step_plan_bytes(projs, n);
  if (need == 0 || plan_bytes < need) return QMM_ERR_SHAPE;
  if (!qmm::aligned(plan, 256)) return QMM_ERR_ALIGN;
  // outputs: disjoint from each other, from the plan and from every input, except that the
  // x of a projection may lie in the outputs of the projection it waits for
  const Range pr = {plan, uint64_t(need)};
  for (int32_t i = 0; i < n; ++i) {
    Range oi[3], ii[5];
    const int no = step_outputs(projs[i], oi);
    const int ni = step_inputs(projs[i], ii);
    for (int a = 0; a < no; ++a) {
      if (overlap(oi[a], pr)) return QMM_ERR_ALIAS;
      for (int b = a + 1; b < no; ++b)
        if (overlap(oi[a], oi[b])) return QMM_ERR_ALIAS;
    }
    for (int b = 0; b < ni; ++b)
      if (overlap(ii[b], pr)) return QMM_ERR_ALIAS;
    for (int32_t j = 0; j < n; ++j) {
      Range oj[3];
      const int noj = step_outputs(projs[j], oj);
      for (int a = 0; a < noj; ++a) {
        if (j > i)
          for (int b = 0; b < no; ++b)
            if (overlap(oj[a], oi[b])) return QMM_ERR_ALIAS;
        for (int b = 0; b < ni; ++b) {
          const bool allowed = b == 0 && projs[i].wait_for == j;
          if (!allowed && overlap(oj[a], ii[b])) return QMM_ERR_ALIAS;
        }
      }
    }
  }
  return qmm::step::build_and_upload(projs, n, plan, need, stream);
}

int qmm_step_run(const qmm_step_proj* projs, int32_t n, const void* plan, hipStream_t stream) {
  if (!projs || !plan) return QMM_ERR_NULL;
  if (n < 1 || n > kMaxStepProjections) return QMM_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    const qmm_step_proj& p = projs[i];
    if ((p.kind != QMM_STEP_LINEAR && p.kind != QMM_STEP_QKV && p.kind != QMM_STEP_GATE_UP_SWIGLU) ||
        p.wait_for < -1 || p.wait_for >= i || !qmm::k_ok(p.K) || p.K <= 512 || p.rows < 1 ||
        p.rows > (int64_t(1) << 30) || !qmm::step::shape_ok(p))
      return QMM_ERR_SHAPE;
    // small launches take the pointers from here, not from the plan
    if (!p.x || !p.codes || !p.scales || !p.biases || !p.out0 ||
        (p.kind == QMM_STEP_QKV && (!p.out1 || !p.out2)))
      return QMM_ERR_NULL;
  }
  if (!qmm::aligned(plan, 256)) return QMM_ERR_ALIGN;
  return qmm::step::launch(projs, n, plan, stream);
}

int qmm_moe_prefill(int stage, const uint16_t* in, int64_t M, int64_t K, const uint32_t* codes,
                    const uint16_t* scales, const uint16_t* biases, int64_t E, int64_t rows,
                    const int32_t* expert_ids, const float* expert_w, int64_t topk, void* workspace,
                    size_t workspace_bytes, void* out, int out_dtype, hipStream_t stream) {
  return qmm::moe_prefill_entry(stage, in, M, K, codes, scales, biases, E, rows, expert_ids, expert_w, topk,
                                workspace, workspace_bytes, nullptr, out, out_dtype, stream);
}

}  // extern "C"

namespace qmm {

int moe_prefill_entry(int stage, const uint16_t* in, int64_t M, int64_t K, const uint32_t* codes,
                      const uint16_t* scales, const uint16_t* biases, int64_t E, int64_t rows,
                      const int32_t* expert_ids, const float* expert_w, int64_t topk, void* workspace,
                      size_t workspace_bytes, void* (*scratch)(size_t), void* out, int out_dtype,
                      hipStream_t stream) {
  const bool route_first = scratch != nullptr;
  if (stage != QMM_MOE_GATE_UP_SWIGLU && stage != QMM_MOE_DOWN_COMBINE) return QMM_ERR_ENUM;
  if (int st = check_weight(in, codes, scales, biases)) return st;
  if (!expert_ids || (!workspace && !route_first) || !out || (stage == QMM_MOE_DOWN_COMBINE && !expert_w))
    return QMM_ERR_NULL;
  if (!out_dtype_ok(out_dtype)) return QMM_ERR_ENUM;
  const bool s1 = stage == QMM_MOE_GATE_UP_SWIGLU;
  const size_t need = qmm_moe_prefill_workspace_bytes(M, topk, E, s1 ? 0 : rows);
  if (need == 0 || !qmm::k_ok(K) || rows < 1 || !codes_fit(rows, K, kU4G64) || (s1 && rows % 2) ||
      !acts_fit(s1 ? M : M * topk, K) || workspace_bytes < need)
    return QMM_ERR_SHAPE;
  // the library's scratch is located only once the sizes are known to fit it
  if (route_first && !(workspace = scratch(need))) return QMM_ERR_LAUNCH;
  const size_t e = out_elem(out_dtype);
  if (!qmm::aligned(out, e) || !qmm::aligned(expert_ids, 4) || (expert_w && !qmm::aligned(expert_w, 4)) ||
      !qmm::aligned(workspace, 256))
    return QMM_ERR_ALIGN;
  const int64_t P = M * topk;
  const int64_t in_elems = s1 ? M * K : P * K;
  const int64_t out_elems = s1 ? P * (rows / 2) : M * rows;
  const Range outs[] = {{out, uint64_t(out_elems) * e}, {workspace, uint64_t(need)}};
  const Range ins[] = {{in, uint64_t(in_elems) * 2},
                       {codes, code_bytes(E * rows, K, kU4G64)},
                       {scales, group_bytes(E * rows, K, kU4G64)},
                       {biases, group_bytes(E * rows, K, kU4G64)},
                       {expert_ids, uint64_t(P) * 4},
                       {expert_w, expert_w ? uint64_t(P) * 4 : 0}};
  if (qmm::any_alias(outs, 2, ins, 6)) return QMM_ERR_ALIAS;

  // A small batch (few pairs: mostly one token per expert) runs the decode gather kernels
  // pair by pair, reading expert_ids directly: stage 1 one SwiGLU GEMV per (token, slot)
  // pair over its expert's rows, stage 2 each token's weighted sum over its slots.  The
  // routing in the workspace is then not read.
  if (P <= kMoePairsByGemv && (s1 || K <= 5120)) {
    qmm::GemvArgs g = {};
    g.x = in;
    g.codes = codes;
    g.scales = scales;
    g.biases = biases;
    g.out0 = out;
    g.K = K;
    g.rows = rows;
    g.I = rows / 2;
    g.expert_ids = expert_ids;
    g.expert_w = expert_w;
    g.E = E;
    g.f32_out = out_dtype == QMM_OUT_F32;
    g.bits = 4;
    g.gshift = kU4G64.gshift;
    if (s1) {
      g.topk = int(P);
      g.moe_div = topk;
      return qmm::launch_moe_gate_up(g, stream);
    }
    g.topk = int(topk);
    g.moe_tokens = M;
    return qmm::launch_moe_down(g, stream);
  }
  // a small batch whose stage 2 the pair-by-pair kernels cannot take (K > 5120): route it
  // here, since qmm_moe_route did not; likewise every call that routes for itself
  if (P <= kMoePairsByGemv || route_first)
    if (int st = qmm::launch_moe_route(expert_ids, M, topk, E, workspace, stream)) return st;

  qmm::GemmArgs a = {};
  a.x = in;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.M = s1 ? M : P;
  a.K = K;
  a.N = rows;
  a.I = rows / 2;
  a.f32_out = out_dtype == QMM_OUT_F32;
  a.bits = 4;
  a.gshift = kU4G64.gshift;
  a.moe_w = s1 ? nullptr : expert_w;
  return qmm::launch_moe_prefill(s1 ? 0 : 1, a, expert_ids, M, topk, E, workspace, out, stream);
}

}  // namespace qmm
