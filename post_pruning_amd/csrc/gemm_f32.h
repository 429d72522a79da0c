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

constexpr int GT = kGemmTile;  // 128 (the default tile; 64 for small contractions)
constexpr int GBK = 32;
constexpr int GS = GBK + 4;    // LDS row stride in floats
constexpr int GTHREADS = 256;
constexpr int GBUF = GT * GS;  // floats per operand buffer of a 128-row tile

// T x T output tile: each of the 4 waves owns a (T/2) x (T/2) sub-tile of
// (T/32) x (T/32) MFMA 16x16 blocks.
template <int T>
struct TileAccT {
  floatx4 v[T / 32][T / 32];
};
using TileAcc = TileAccT<GT>;

template <int T>
__device__ inline void tile_zero(TileAccT<T>& a) {
#pragma unroll
  for (int i = 0; i < T / 32; ++i)
#pragma unroll
    for (int j = 0; j < T / 32; ++j) a.v[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// Output element held by (lane, i, j, v): row / column inside the T x T tile.
template <int T = GT>
__device__ inline int tile_row(int wave, int lane, int i, int v) {
  return (wave >> 1) * (T / 2) + i * 16 + (lane >> 4) * 4 + v;
}
template <int T = GT>
__device__ inline int tile_col(int wave, int lane, int j) {
  return (wave & 1) * (T / 2) + j * 16 + (lane & 15);
}

// acc += P[0:T, 0:32] * Q[0:T, 0:32]^T from LDS tiles [T][GS].
template <int T>
__device__ inline void tile_mma_chunk(TileAccT<T>& acc, const float* Pl, const float* Ql, int wave,
                                      int lane) {
  constexpr int NI = T / 32;
  const int prow = (wave >> 1) * (T / 2) + (lane & 15);
  const int qrow = (wave & 1) * (T / 2) + (lane & 15);
#pragma unroll
  for (int g = 0; g < GBK / 16; ++g) {
    const int k = g * 16 + (lane >> 4) * 4;
    floatx4 p[NI], q[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) p[i] = *reinterpret_cast<const floatx4*>(Pl + (prow + i * 16) * GS + k);
#pragma unroll
    for (int j = 0; j < NI; ++j) q[j] = *reinterpret_cast<const floatx4*>(Ql + (qrow + j * 16) * GS + k);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[i][e], q[j][e], acc.v[i][j], 0, 0, 0);
  }
}

// Rows of a k-contiguous fp32 matrix: element (r, k) = scale * src[r*ld + k],
// valid for r < rows, k < kend (rows >= 1, kend >= 1).
template <int T>
struct RowsF32T {
  const float* src;
  int64_t ld;
  int rows;
  int64_t kend;
  float scale;
  float v[T / 8];
  __device__ inline void load(int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const int64_t k = k0 + kk;
    const int64_t kc = k < kend ? k : kend - 1;
#pragma unroll
    for (int rr = 0; rr < T / 8; ++rr) {
      const int r = r0 + rr * 8;
      const int rc = r < rows ? r : rows - 1;
      v[rr] = src[(int64_t)rc * ld + kc];
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const bool kok = k0 + kk < kend;
#pragma unroll
    for (int rr = 0; rr < T / 8; ++rr) {
      const int r = r0 + rr * 8;
      lds[r * GS + kk] = (r < rows && kok) ? v[rr] * scale : 0.f;
    }
  }
};
using RowsF32 = RowsF32T<GT>;

// Rows of a k-contiguous fp32 matrix with 16-byte aligned rows (ld % 4 == 0,
// aligned base): T/32 16-byte loads per thread per chunk (8 threads per row,
// rows r0, r0 + 32, ...), written to LDS with 16-byte stores.  Element (r, k)
// = src[r*ld + k], valid for r < rows, k < kend (kend % 4 == 0).
template <int T>
struct RowsF32VT {
  const float* src;
  int64_t ld;
  int rows;
  int64_t kend;
  floatx4 v[T / 32];
  __device__ inline void load(int64_t k0) {
    const int k4 = (threadIdx.x & 7) * 4, r0 = threadIdx.x >> 3;
    const int64_t k = k0 + k4;
    const int64_t kc = k < kend ? k : kend - 4;
#pragma unroll
    for (int u = 0; u < T / 32; ++u) {
      const int r = r0 + 32 * u;
      const int rc = r < rows ? r : rows - 1;
      v[u] = *reinterpret_cast<const floatx4*>(src + (int64_t)rc * ld + kc);
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int k4 = (threadIdx.x & 7) * 4, r0 = threadIdx.x >> 3;
    const bool kok = k0 + k4 < kend;
#pragma unroll
    for (int u = 0; u < T / 32; ++u) {
      const int r = r0 + 32 * u;
      *reinterpret_cast<floatx4*>(&lds[r * GS + k4]) =
          (r < rows && kok) ? v[u] : floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
};
using RowsF32V = RowsF32VT<GT>;

// Row-major [k][j] fp32 read transposed (any alignment): thread t owns column
// j = t % T and KT = 32 T / 256 consecutive k of the chunk.  Its loads are
// 4-byte but coalesced across the wave (consecutive j); it writes its k-values
// to LDS with 16-byte stores into row j, which with the 144-byte row stride
// land in distinct bank groups for every 16 consecutive lanes.
// Element (j, k) = src[k*ld + j], valid for j < cols, k < kend.
template <int T>
struct ColsF32TT {
  static constexpr int KT = GBK * T / GTHREADS;  // 16 (T = 128) or 8 (T = 64)
  const float* src;
  int64_t ld;
  int cols;
  int64_t kend;
  float v[KT];
  __device__ inline void load(int64_t k0) {
    const int j = threadIdx.x % T, kb = (threadIdx.x / T) * KT;
    const int jc = j < cols ? j : cols - 1;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      const int64_t k = k0 + kb + u;
      const int64_t kc = k < kend ? k : kend - 1;
      v[u] = src[kc * ld + jc];
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int j = threadIdx.x % T, kb = (threadIdx.x / T) * KT;
#pragma unroll
    for (int q = 0; q < KT / 4; ++q) {
      floatx4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (j < cols && k0 + kb + 4 * q + e < kend) ? v[4 * q + e] : 0.f;
      *reinterpret_cast<floatx4*>(&lds[j * GS + kb + 4 * q]) = t;
    }
  }
};
using ColsF32T = ColsF32TT<GT>;

// acc += P * Q^T over k in [0, K): P and Q loaders with the load/store
// interface above; lds holds 4 * T * GS floats (two buffers per operand).
template <int T, class PL, class QL>
__device__ inline void tile_gemm_pipelined(TileAccT<T>& acc, PL& pl, QL& ql, int64_t K, float* lds) {
  constexpr int BUF = T * GS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nch = ceil_div(K, GBK);
  if (nch <= 0) return;
  pl.load(0);
  ql.load(0);
  pl.store(lds, 0);
  ql.store(lds + BUF, 0);
  __syncthreads();
  for (int64_t c = 0; c < nch; ++c) {
    float* cur = lds + (c & 1) * 2 * BUF;
    float* nxt = lds + ((c + 1) & 1) * 2 * BUF;
    const bool more = c + 1 < nch;
    if (more) {
      pl.load((c + 1) * GBK);
      ql.load((c + 1) * GBK);
    }
    tile_mma_chunk(acc, cur, cur + BUF, wave, lane);
    if (more) {
      pl.store(nxt, (c + 1) * GBK);
      ql.store(nxt + BUF, (c + 1) * GBK);
    }
    __syncthreads();
  }
}

// C[0:rows, 0:cols] -= acc (C row-major with leading dimension ldc), staged
// through LDS (which must hold T * (T + 4) floats and be free) so that the
// read-modify-write of C is done with float4 accesses, T/4 lanes per row.
// Epilogue hook: called with (row, column, new value) of every element the
// epilogue stores; the default does nothing.
struct NoHook {
  __device__ void operator()(int, int, float) const {}
};

// A T x T tile of C read ahead of the contraction that updates it (the
// loads are in flight while the products are formed).  Applies when the tile
// is full width with 16-byte aligned rows, the layout of tile_sub_from's
// vector path: thread t holds columns 4 (t % (T/4)) .. +3 of rows
// t / (T/4) + RPP * rr.
template <int T>
struct CTileV {
  static constexpr int RPP = GTHREADS / (T / 4);
  floatx4 cv[T / RPP];
  __device__ static bool ok(const float* C, int64_t ldc, int cols) {
    return (cols == T) && ((ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
  }
  __device__ inline void load(const float* __restrict__ C, int64_t ldc, int rows) {
    const int c4 = (threadIdx.x % (T / 4)) * 4, r0 = threadIdx.x / (T / 4);
#pragma unroll
    for (int rr = 0; rr < T / RPP; ++rr) {
      const int r = r0 + rr * RPP;
      const int rc = r < rows ? r : rows - 1;
      cv[rr] = *reinterpret_cast<const floatx4*>(C + (int64_t)rc * ldc + c4);
    }
  }
};

// C -= acc with C's values read ahead into ct (CTileV::ok held); the
// accumulator goes through LDS as in tile_sub_from.
template <int T, class Hook = NoHook>
__device__ inline void tile_sub_pre(float* __restrict__ C, int64_t ldc, int rows, const CTileV<T>& ct,
                                    const TileAccT<T>& acc, float* lds, const Hook& hook = Hook()) {
  constexpr int TS = T + 4;
  constexpr int RPP = CTileV<T>::RPP;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < T / 32; ++i)
#pragma unroll
    for (int jj = 0; jj < T / 32; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        lds[tile_row<T>(wave, lane, i, v) * TS + tile_col<T>(wave, lane, jj)] = acc.v[i][jj][v];
  __syncthreads();
  const int c4 = (threadIdx.x % (T / 4)) * 4, r0 = threadIdx.x / (T / 4);
#pragma unroll
  for (int rr = 0; rr < T / RPP; ++rr) {
    const int r = r0 + rr * RPP;
    if (r < rows) {
      const floatx4 t = *reinterpret_cast<const floatx4*>(&lds[r * TS + c4]);
      const floatx4 nv = ct.cv[rr] - t;
      *reinterpret_cast<floatx4*>(C + (int64_t)r * ldc + c4) = nv;
#pragma unroll
      for (int e = 0; e < 4; ++e) hook(r, c4 + e, nv[e]);
    }
  }
}

template <int T, class Hook = NoHook>
__device__ inline void tile_sub_from(float* __restrict__ C, int64_t ldc, int rows, int cols,
                                     const TileAccT<T>& acc, float* lds, const Hook& hook = Hook()) {
  constexpr int TS = T + 4;
  constexpr int RPP = GTHREADS / (T / 4);  // rows per pass
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < T / 32; ++i)
#pragma unroll
    for (int jj = 0; jj < T / 32; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        lds[tile_row<T>(wave, lane, i, v) * TS + tile_col<T>(wave, lane, jj)] = acc.v[i][jj][v];
  __syncthreads();
  const int c4 = (threadIdx.x % (T / 4)) * 4;
  const int r0 = threadIdx.x / (T / 4);
  const bool vec = (cols == T) && ((ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
  if (vec) {
    // all loads first (C may alias nothing else, but the compiler cannot know
    // that a store does not feed a later load), then subtract and store
    floatx4 cv[T / RPP];
#pragma unroll
    for (int rr = 0; rr < T / RPP; ++rr) {
      const int r = r0 + rr * RPP;
      const int rc = r < rows ? r : rows - 1;
      cv[rr] = *reinterpret_cast<const floatx4*>(C + (int64_t)rc * ldc + c4);
    }
#pragma unroll
    for (int rr = 0; rr < T / RPP; ++rr) {
      const int r = r0 + rr * RPP;
      if (r < rows) {
        const floatx4 t = *reinterpret_cast<const floatx4*>(&lds[r * TS + c4]);
        const floatx4 nv = cv[rr] - t;
        *reinterpret_cast<floatx4*>(C + (int64_t)r * ldc + c4) = nv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hook(r, c4 + e, nv[e]);
      }
    }
  } else {
    for (int rr = 0; rr < T / RPP; ++rr) {
      const int r = r0 + rr * RPP;
      if (r >= rows) break;
      const floatx4 t = *reinterpret_cast<const floatx4*>(&lds[r * TS + c4]);
      float* crow = C + (int64_t)r * ldc;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c4 + e < cols) {
          const float nv = crow[c4 + e] - t[e];
          crow[c4 + e] = nv;
          hook(r, c4 + e, nv);
        }
    }
  }
}

}  // namespace sg
