// Host-side argument checks for the C ABI (see qmm_validate.h).
#include "qmm_validate.h"

#include "qmm.h"

namespace qmm {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static bool overlap(const Range& a, const Range& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool any_alias(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
  }
  return false;
}

bool k_ok(int64_t K) { return K >= 64 && K % 64 == 0 && K <= QMM_MAX_K; }

}  // namespace qmm
