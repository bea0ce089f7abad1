// Argument validation for the C ABI: pure host C++, no HIP calls, so it runs (and
// is tested) without a GPU.  Every check happens before anything is enqueued.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace qmm {

struct Range {
  const void* p;
  uint64_t bytes;
};

bool aligned(const void* p, size_t a);
// Any overlap between two outputs, or between an output and an input.
bool any_alias(const Range* outs, int n_out, const Range* ins, int n_in);
// K >= 64, K % 64 == 0, K <= QMM_MAX_K.
bool k_ok(int64_t K);

}  // namespace qmm
