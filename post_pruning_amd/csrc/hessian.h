// Hessian accumulation: launch plan and entry points (H += Xc^T Xc).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sg.h"

namespace sg {

constexpr int kHessTileRows = 256;  // Hessian output tile: rows (one row panel)
constexpr int kHessTileCols = 384;  // and columns (one column panel)

constexpr int kHessMaxSplits = 64;

// Token ranges of the splits: split s covers tokens [b[s], b[s + 1]).
struct HessSplits {
  int64_t b[kHessMaxSplits + 1];
};

struct HessPlan {
  int64_t tiles;       // 256x384 tiles covering the lower triangle
  int splits;          // token splits
  HessSplits bounds;   // their token ranges (b[splits] = T)
  int group;           // tile-panel group edge of the per-XCD tile order
  int64_t grid;        // workgroups launched (8 equal per-XCD shares)
  size_t part_bytes;   // split counters + partial tiles (0 without splits)
  int sync_rounds;     // lockstep rounds per XCD
  bool sync;           // lockstep counters fit in the workspace
  size_t ws_bytes;     // partials + split counters + lockstep counters
};
HessPlan hessian_plan(int64_t n, int64_t T, size_t ws_avail, bool limit_by_ws);
sg_status launch_hessian_bf16(float* H, int64_t n, const uint16_t* X, int64_t T,
                              int64_t ldx, const HessPlan& plan, void* ws,
                              hipStream_t st);
sg_status launch_hessian_f32(float* H, int64_t n, const float* X, int64_t T,
                             int64_t ldx, hipStream_t st);

}  // namespace sg
