// fp32 MFMA tile core for the dense contractions of the solver: the trailing
// updates of the blocked factorisation, the lazy trailing update of the column
// sweep, and the reconstruction error.
//
// One 256-thread workgroup owns a 128x128 output tile; its 4 waves form a 2x2
// grid of 64x64 sub-tiles, each a 4x4 array of v_mfma_f32_16x16x4_f32.
// Operands are staged in LDS 32 k-values at a time with k contiguous in every
// LDS row ([row][k], row stride 36 floats = 144 B, conflict-free for the
// 16-byte fragment reads), so a lane fetches 4 consecutive k-values of its
// row with one ds_read_b128 and feeds them to 4 MFMAs.  A and B use the same
// lane -> k assignment, so the k permutation inside a 16-wide group cancels.
#pragma once

#include "sg_internal.h"

namespace sg {

constexpr int GT = kGemmTile;  // 128
constexpr int GBK = 32;
constexpr int GS = GBK + 4;    // LDS row stride in floats
constexpr int GTHREADS = 256;

struct TileAcc {
  floatx4 v[4][4];
};

__device__ inline void tile_zero(TileAcc& a) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) a.v[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// Output element held by (lane, i, j, v): row / column inside the 128x128 tile.
__device__ inline int tile_row(int wave, int lane, int i, int v) {
  return (wave >> 1) * 64 + i * 16 + (lane >> 4) * 4 + v;
}
__device__ inline int tile_col(int wave, int lane, int j) {
  return (wave & 1) * 64 + j * 16 + (lane & 15);
}

// acc += P[0:128, 0:32] * Q[0:128, 0:32]^T from LDS tiles [128][GS].
__device__ inline void tile_mma_chunk(TileAcc& acc, const float* Pl, const float* Ql, int wave,
                                      int lane) {
  const int prow = (wave >> 1) * 64 + (lane & 15);
  const int qrow = (wave & 1) * 64 + (lane & 15);
#pragma unroll
  for (int g = 0; g < GBK / 16; ++g) {
    const int k = g * 16 + (lane >> 4) * 4;
    floatx4 p[4], q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = *reinterpret_cast<const floatx4*>(Pl + (prow + i * 16) * GS + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = *reinterpret_cast<const floatx4*>(Ql + (qrow + j * 16) * GS + k);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[i][e], q[j][e], acc.v[i][j], 0, 0, 0);
  }
}

// Stage rows of a k-contiguous fp32 matrix: lds[r][kk] = scale * src[r*ld + k0 + kk]
// for r < rows, k0 + kk < kend (zero elsewhere; rows >= 1 and kend > k0).
// All loads are issued first from clamped in-bounds addresses, then the
// out-of-range values are zeroed as they are written, so the loads overlap.
__device__ inline void stage_rows_f32(float* lds, const float* __restrict__ src, int64_t ld,
                                      int rows, int64_t k0, int64_t kend, float scale = 1.f) {
  const int kk = threadIdx.x & 31;
  const int r0 = threadIdx.x >> 5;
  const int64_t k = k0 + kk;
  const int64_t kc = k < kend ? k : kend - 1;
  float v[GT / 8];
#pragma unroll
  for (int rr = 0; rr < GT / 8; ++rr) {
    const int r = r0 + rr * 8;
    const int rc = r < rows ? r : rows - 1;
    v[rr] = src[(int64_t)rc * ld + kc];
  }
#pragma unroll
  for (int rr = 0; rr < GT / 8; ++rr) {
    const int r = r0 + rr * 8;
    lds[r * GS + kk] = (r < rows && k < kend) ? v[rr] * scale : 0.f;
  }
}

// Stage a row-major [k][j] fp32 matrix transposed: lds[j][kk] = src[(k0+kk)*ld + j]
// for j < cols, k0 + kk < kend (zero elsewhere; cols >= 1 and kend > k0).
__device__ inline void stage_cols_f32(float* lds, const float* __restrict__ src, int64_t ld,
                                      int cols, int64_t k0, int64_t kend) {
  const int j = threadIdx.x & 127;
  const int kh = threadIdx.x >> 7;
  const int jc = j < cols ? j : cols - 1;
  float v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t k = k0 + kh * 16 + u;
    const int64_t kc = k < kend ? k : kend - 1;
    v[u] = src[kc * ld + jc];
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int kk = kh * 16 + u;
    lds[j * GS + kk] = (j < cols && k0 + kk < kend) ? v[u] : 0.f;
  }
}

}  // namespace sg
