// qmm_moe_prefill_noalloc: one stage of the routed experts over a batch of tokens, as
// qmm_moe_prefill, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).  The routing tables and
// the stage-2 products, which qmm_moe_prefill keeps in a caller workspace, live here in a
// file-scope device array of QMM_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process
// ends; each call buckets expert_ids into it itself before running the stage.
//
// In host code `scratch` names a host-side stand-in, not device memory: the array's device
// address is looked up once per device (hipGetSymbolAddress, with that device current) on
// the first call there, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qmm.h"
#include "qmm_internal.h"

namespace {

constexpr size_t kScratchBytes = QMM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of this device's scratch array (null if it cannot be located).
void* scratch_addr(size_t) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_addr[dev] = p;
  }
  return g_addr[dev];
}

}  // namespace

extern "C" int qmm_moe_prefill_noalloc(int stage, const uint16_t* in, int64_t M, int64_t K, const uint32_t* codes,
                                       const uint16_t* scales, const uint16_t* biases, int64_t E, int64_t rows,
                                       const int32_t* expert_ids, const float* expert_w, int64_t topk, void* out,
                                       int out_dtype, hipStream_t stream) {
  return qmm::moe_prefill_entry(stage, in, M, K, codes, scales, biases, E, rows, expert_ids, expert_w, topk, nullptr,
                                kScratchBytes, scratch_addr, out, out_dtype, stream);
}
