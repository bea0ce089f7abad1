// Layout of a decode-step plan (qmm_step_plan / qmm_step_run): several 4-bit group-64
// projections of one token, each computed with the per-call decode arithmetic for its K.
//
// The projections are grouped into launches.  A projection's level is 0 if it reads no other
// projection's output, else one more than the level of the projection it reads; the
// projections of one level whose K fits one wave (K <= 5120) share one launch of the
// single-slice kernel, those whose K is split over 8 or 16 waves one launch of the K-split
// kernel per split.  Launches run in order of (level, kind), so a projection starts after
// every projection it reads has finished, and no launch synchronises inside itself.
//
// A launch's work is a list of positions over its projections (in projection order):
//   * single-slice launch: one position per row unit (two rows; for gate+up one (gate, up)
//     row pair), each wave taking one contiguous range of positions;
//   * K-split launch: one position per row unit, each block of ks waves taking a contiguous
//     range of units, wave s computing K slice s, the slices added in LDS in wave order.
#pragma once
#include <stdint.h>

namespace qmm {
namespace step {

constexpr uint32_t kMagic = 0x51535450u;  // "QSTP"
constexpr int kWavesPerBlockSingle = 4;

// Single-slice launches; K split over 8 waves with at most 4 chunks per lane (K <= 32768) or
// with 5 (K <= 40960; more registers, so fewer blocks per CU); K split over 16 waves.
enum LaunchKind : int32_t { kSingle = 0, kSplit8 = 1, kSplit8Wide = 2, kSplit16 = 3 };

struct Proj {
  const uint16_t* x;         // [K] bf16
  const uint32_t* codes;     // [rows][K/8]
  const uint16_t* scales;    // [rows][K/64]
  const uint16_t* biases;    // [rows][K/64]
  const uint16_t* lin_bias;  // nullable [rows]
  void* out0;                // QKV routing: rows [0, q_out); SWIGLU: h
  void* out1;                // QKV routing: rows [q_out, q_out + kv_out)
  void* out2;                // QKV routing: the rest
  int32_t K, rows, q_out, kv_out, I;  // a plain projection has q_out = rows, kv_out = 0
  int32_t epi;               // EPI_QKV (plain projections too) or EPI_SWIGLU
  int32_t f32_out;
  int32_t ks, cpl;           // K slices (1, 8 or 16) and 32-code chunks per lane in a slice
  int32_t units;             // row units
};

struct Seg {
  int64_t begin;  // first position of the projection in its launch's list
  int32_t proj;
  int32_t pad;
};

// One launch: segments [seg0, seg0 + n_seg) of the plan's segment array, followed by a
// sentinel whose begin is the launch's position count.
struct Launch {
  int32_t kind;
  int32_t seg0;
  int32_t n_seg;
  int32_t blocks;   // grid size
  int64_t total;
  int64_t blk0;     // first BlockSegs entry of this launch
};

// Per launch, per block: the segment of the block's first position and of its last (the
// projections whose activations a single-slice block stages), at the launch's grid size.
struct BlockSegs {
  int32_t first, last;
};

// A launch of at most kInlineProjs projections, passed by value as its kernel's argument:
// its projections in launch order and their first positions, begin[n_seg] (and the unused
// entries after it) the launch's position count.
constexpr int kInlineProjs = 4;
struct InlineLaunch {
  Proj projs[kInlineProjs];
  int64_t begin[kInlineProjs + 1];
  int32_t n_seg;
  int32_t pad;
};

struct Header {
  uint32_t magic;
  int32_t n_proj;
  int32_t n_launch;
  int32_t pad;
  uint64_t proj_off;    // byte offsets from the plan's start
  uint64_t launch_off;
  uint64_t seg_off;
  uint64_t blk_off;     // BlockSegs of every launch's blocks, launch after launch
  uint64_t bytes;       // plan size
};

}  // namespace step
}  // namespace qmm
