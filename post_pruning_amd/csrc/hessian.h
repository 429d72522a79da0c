// Hessian accumulation: launch plan and entry points (H += Xc^T Xc).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sg.h"

namespace sg {

constexpr int kHessTile = 256;    // Hessian output tile edge

struct HessPlan {
  int64_t tiles;       // lower-triangle 256x256 tiles
  int splits;          // token splits
  int64_t tok_per_split;
  int group;           // tile-panel group edge of the per-XCD tile order
  int64_t grid;        // workgroups launched (8 equal per-XCD shares)
  size_t ws_bytes;     // partials + counters
};
HessPlan hessian_plan(int64_t n, int64_t T, size_t ws_avail, bool limit_by_ws);
sg_status launch_hessian_bf16(float* H, int64_t n, const uint16_t* X, int64_t T,
                              int64_t ldx, const HessPlan& plan, void* ws,
                              hipStream_t st);
sg_status launch_hessian_f32(float* H, int64_t n, const float* X, int64_t T,
                             int64_t ldx, hipStream_t st);

}  // namespace sg
