// Device side of the fused QKV epilogue with rotary position embedding (EPI_ROPE): which
// two weight rows rotate together, and the rotation + split store of one such pair.
//
// The pages' unshipped second phase fuses the split of the QKV output with its rotary
// embedding ("Sanctum-MLX", shipped phases table, Phase 2; "The Cathedral Doubled Itself",
// the kernel that worked and the kernel that won't).  The rotation is the half-split form
// over the first `rot` dims of each Q and K head: dims i and i + rot/2 turn together by
// the angle of table column i at the token's position.  The dims past `rot` pass through,
// paired (rot + j, rot + j + (head_dim - rot)/2) only so that every unit of the kernels
// holds two rows; V and output-gate heads pass through the same way.
#pragma once
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

enum RopeBuf : int { ROPE_Q = 0, ROPE_K = 1, ROPE_V = 2, ROPE_GATE = 3 };

struct RopePair {
  int32_t ra, rb;  // weight rows of the pair
  int32_t buf;     // RopeBuf
  int32_t head;    // head within its output
  int32_t da, db;  // dims within the head
  int32_t ri;      // table column of the rotation, -1 if the pair passes through
};

// Pair p (0 <= p < rows/2) of the fused weight.
__device__ __forceinline__ RopePair rope_pair(uint32_t p, const RopeArgs& g) {
  const uint32_t hd = uint32_t(g.head_dim), half = hd >> 1, rh = uint32_t(g.rot) >> 1;
  const uint32_t h = p / half;
  const uint32_t i = p - h * half;
  RopePair r;
  if (i < rh) {
    r.da = int32_t(i);
    r.db = int32_t(i + rh);
    r.ri = int32_t(i);
  } else {
    const uint32_t j = i - rh;
    r.da = int32_t(uint32_t(g.rot) + j);
    r.db = int32_t(uint32_t(g.rot) + j + ((hd - uint32_t(g.rot)) >> 1));
    r.ri = -1;
  }
  r.ra = int32_t(h * hd) + r.da;
  r.rb = int32_t(h * hd) + r.db;
  const uint32_t qsec = uint32_t(g.n_q) << g.q_gate;  // heads of the Q section
  if (h < qsec) {
    r.buf = (g.q_gate && (h & 1)) ? ROPE_GATE : ROPE_Q;
    r.head = int32_t(h >> g.q_gate);
  } else if (h < qsec + uint32_t(g.n_kv)) {
    r.buf = ROPE_K;
    r.head = int32_t(h - qsec);
  } else {
    r.buf = ROPE_V;
    r.head = int32_t(h - qsec - uint32_t(g.n_kv));
  }
  if (r.buf == ROPE_V || r.buf == ROPE_GATE) r.ri = -1;
  return r;
}

// Rotates the pair's values (va at dim da, vb at dim db) of token m by (c, s), if the pair
// rotates, and stores both into their head of q/k/v/gate.  (a, b) -> (a c - b s, b c + a s)
// in fp32.
__device__ __forceinline__ void rope_store_cs(const RopeArgs& g, void* q, void* k, void* v, const RopePair& r,
                                              int64_t m, float va, float vb, float c, float s, bool f32) {
  if (r.ri >= 0) {
    const float a = va, b = vb;
    va = fmaf(a, c, -(b * s));
    vb = fmaf(b, c, a * s);
  }
  void* dst;
  int64_t nh;
  switch (r.buf) {
    case ROPE_Q: dst = q; nh = g.n_q; break;
    case ROPE_K: dst = k; nh = g.n_kv; break;
    case ROPE_V: dst = v; nh = g.n_kv; break;
    default: dst = g.gate; nh = g.n_q; break;
  }
  const int64_t base = (m * nh + r.head) * int64_t(g.head_dim);
  store_out(dst, base + r.da, va, f32);
  store_out(dst, base + r.db, vb, f32);
}

// The same, reading c and s from the table at the token's (clamped) position.
__device__ __forceinline__ void rope_store(const RopeArgs& g, void* q, void* k, void* v, const RopePair& r,
                                           int64_t m, float va, float vb, bool f32) {
  float c = 1.f, s = 0.f;
  if (r.ri >= 0) {
    const int32_t pos = min(max(g.positions[m], 0), g.max_pos - 1);
    const float* t = g.cos_sin + int64_t(pos) * g.rot;
    c = t[r.ri];
    s = t[(g.rot >> 1) + r.ri];
  }
  rope_store_cs(g, q, k, v, r, m, va, vb, c, s, f32);
}

}  // namespace qmm
