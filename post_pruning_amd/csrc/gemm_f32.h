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
//
// The k loop is software-pipelined: chunk c+1 is loaded into registers while
// chunk c is multiplied out of one of two LDS buffers, so global-memory latency
// hides behind the MFMAs.  Loads always use clamped in-bounds addresses and
// out-of-range values are zeroed when they are written to LDS, so a chunk's
// loads are issued back to back without waits in between.
#pragma once

#include "sg_internal.h"

namespace sg {

constexpr int GT = kGemmTile;  // 128
constexpr int GBK = 32;
constexpr int GS = GBK + 4;    // LDS row stride in floats
constexpr int GTHREADS = 256;
constexpr int GBUF = GT * GS;  // floats per operand buffer

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

// Rows of a k-contiguous fp32 matrix: element (r, k) = scale * src[r*ld + k],
// valid for r < rows, k < kend (rows >= 1, kend >= 1).
struct RowsF32 {
  const float* src;
  int64_t ld;
  int rows;
  int64_t kend;
  float scale;
  float v[GT / 8];
  __device__ inline void load(int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const int64_t k = k0 + kk;
    const int64_t kc = k < kend ? k : kend - 1;
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      const int rc = r < rows ? r : rows - 1;
      v[rr] = src[(int64_t)rc * ld + kc];
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const bool kok = k0 + kk < kend;
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      lds[r * GS + kk] = (r < rows && kok) ? v[rr] * scale : 0.f;
    }
  }
};

// A row-major [k][j] fp32 matrix read transposed: element (j, k) = src[k*ld + j],
// valid for j < cols, k < kend (cols >= 1, kend >= 1).
struct ColsF32 {
  const float* src;
  int64_t ld;
  int cols;
  int64_t kend;
  float v[16];
  __device__ inline void load(int64_t k0) {
    const int j = threadIdx.x & 127, kh = threadIdx.x >> 7;
    const int jc = j < cols ? j : cols - 1;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t k = k0 + kh * 16 + u;
      const int64_t kc = k < kend ? k : kend - 1;
      v[u] = src[kc * ld + jc];
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int j = threadIdx.x & 127, kh = threadIdx.x >> 7;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int kk = kh * 16 + u;
      lds[j * GS + kk] = (j < cols && k0 + kk < kend) ? v[u] : 0.f;
    }
  }
};

// Rows of a k-contiguous fp32 matrix with 16-byte aligned rows (ld % 4 == 0,
// aligned base): four 16-byte loads per thread per chunk (8 threads per row,
// rows r0, r0 + 32, ...), written to LDS with 16-byte stores.  Element (r, k)
// = src[r*ld + k], valid for r < rows, k < kend (kend % 4 == 0).
struct RowsF32V {
  const float* src;
  int64_t ld;
  int rows;
  int64_t kend;
  floatx4 v[4];
  __device__ inline void load(int64_t k0) {
    const int k4 = (threadIdx.x & 7) * 4, r0 = threadIdx.x >> 3;
    const int64_t k = k0 + k4;
    const int64_t kc = k < kend ? k : kend - 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + 32 * u;
      const int rc = r < rows ? r : rows - 1;
      v[u] = *reinterpret_cast<const floatx4*>(src + (int64_t)rc * ld + kc);
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int k4 = (threadIdx.x & 7) * 4, r0 = threadIdx.x >> 3;
    const bool kok = k0 + k4 < kend;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + 32 * u;
      *reinterpret_cast<floatx4*>(&lds[r * GS + k4]) =
          (r < rows && kok) ? v[u] : floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Row-major [k][j] fp32 read transposed with 16-byte aligned rows (ld % 4 ==
// 0, aligned base, cols % 4 == 0): thread t loads columns 4*(t%32) .. +3 of
// rows k = t/32 + 8u (u < 4) with four 16-byte loads; element (j, k) =
// src[k*ld + j], valid for j < cols, k < kend.
struct ColsF32V {
  const float* src;
  int64_t ld;
  int cols;
  int64_t kend;
  floatx4 v[4];
  __device__ inline void load(int64_t k0) {
    const int j4 = (threadIdx.x & 31) * 4, kh = threadIdx.x >> 5;
    const int jc = j4 < cols ? j4 : cols - 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t k = k0 + kh + 8 * u;
      const int64_t kc = k < kend ? k : kend - 1;
      v[u] = *reinterpret_cast<const floatx4*>(src + kc * ld + jc);
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int j4 = (threadIdx.x & 31) * 4, kh = threadIdx.x >> 5;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = kh + 8 * u;
      const bool ok = j4 < cols && k0 + kk < kend;
#pragma unroll
      for (int e = 0; e < 4; ++e) lds[(j4 + e) * GS + kk] = ok ? v[u][e] : 0.f;
    }
  }
};

// acc += P * Q^T over k in [0, K): P and Q loaders with the load/store
// interface above; lds holds 4 * GBUF floats (two buffers per operand).
template <class PL, class QL>
__device__ inline void tile_gemm_pipelined(TileAcc& acc, PL& pl, QL& ql, int64_t K, float* lds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nch = ceil_div(K, GBK);
  if (nch <= 0) return;
  pl.load(0);
  ql.load(0);
  pl.store(lds, 0);
  ql.store(lds + GBUF, 0);
  __syncthreads();
  for (int64_t c = 0; c < nch; ++c) {
    float* cur = lds + (c & 1) * 2 * GBUF;
    float* nxt = lds + ((c + 1) & 1) * 2 * GBUF;
    const bool more = c + 1 < nch;
    if (more) {
      pl.load((c + 1) * GBK);
      ql.load((c + 1) * GBK);
    }
    tile_mma_chunk(acc, cur, cur + GBUF, wave, lane);
    if (more) {
      pl.store(nxt, (c + 1) * GBK);
      ql.store(nxt + GBUF, (c + 1) * GBK);
    }
    __syncthreads();
  }
}

// C[0:rows, 0:cols] -= acc (C row-major with leading dimension ldc), staged
// through LDS (which must hold GT * (GT + 4) floats and be free) so that the
// read-modify-write of C is done with float4 accesses, 32 lanes per row.
__device__ inline void tile_sub_from(float* __restrict__ C, int64_t ldc, int rows, int cols,
                                     const TileAcc& acc, float* lds) {
  constexpr int TS = GT + 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        lds[tile_row(wave, lane, i, v) * TS + tile_col(wave, lane, jj)] = acc.v[i][jj][v];
  __syncthreads();
  const int c4 = (threadIdx.x & 31) * 4;
  const int r0 = threadIdx.x >> 5;
  const bool vec = (cols == GT) && ((ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
  if (vec) {
    // all loads first (C may alias nothing else, but the compiler cannot know
    // that a store does not feed a later load), then subtract and store
    floatx4 cv[GT / 8];
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      const int rc = r < rows ? r : rows - 1;
      cv[rr] = *reinterpret_cast<const floatx4*>(C + (int64_t)rc * ldc + c4);
    }
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      if (r < rows) {
        const floatx4 t = *reinterpret_cast<const floatx4*>(&lds[r * TS + c4]);
        *reinterpret_cast<floatx4*>(C + (int64_t)r * ldc + c4) = cv[rr] - t;
      }
    }
  } else {
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      if (r >= rows) break;
      const floatx4 t = *reinterpret_cast<const floatx4*>(&lds[r * TS + c4]);
      float* crow = C + (int64_t)r * ldc;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c4 + e < cols) crow[c4 + e] -= t[e];
    }
  }
}

}  // namespace sg
