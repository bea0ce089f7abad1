// Host-only test shim: exposes the C ABI's argument checks (qmm_validate.cpp) with C
// linkage so the CPU tests can drive them through ctypes without a GPU.  Built by
// tests/test_abi.py with g++ together with qmm_validate.cpp; never part of libqmm.so.
#include "qmm_validate.h"

extern "C" {
int shim_aligned(const void* p, unsigned long a) { return qmm::aligned(p, a) ? 1 : 0; }
int shim_k_ok(long long K) { return qmm::k_ok(K) ? 1 : 0; }
// outs/ins: arrays of (pointer, bytes) pairs.
int shim_any_alias(const unsigned long long* outs, int n_out, const unsigned long long* ins, int n_in) {
  qmm::Range o[8], i[8];
  for (int k = 0; k < n_out; ++k) o[k] = qmm::Range{reinterpret_cast<const void*>(outs[2 * k]), outs[2 * k + 1]};
  for (int k = 0; k < n_in; ++k) i[k] = qmm::Range{reinterpret_cast<const void*>(ins[2 * k]), ins[2 * k + 1]};
  return qmm::any_alias(o, n_out, i, n_in) ? 1 : 0;
}
}
