// fp32-accurate tile core on bf16 MFMA for the dense contractions of the
// solver (the lazy trailing update and the factorisation's trailing updates).
//
// Every fp32 operand value x is split exactly into three bf16 parts,
//   h = bf16(x), m = bf16(x - h), l = bf16(x - h - m),   x = h + m + l
// (round to nearest even at each step; 3 x 8 significand bits hold the 24 of
// fp32).  A product x*y is formed from the six terms that reach the fp32
// rounding level, hh + hm + mh + hl + lh + mm (the dropped ml, lm, ll are
// below 2^-24 relative), each exact in the fp32 accumulator of
// v_mfma_f32_16x16x32_bf16.  Six bf16 MFMAs of K = 32 replace eight fp32
// MFMAs of K = 4, at twice the rate each: 2.7x the fp32 MFMA throughput.
// This is the six-product ("bf16x6") scheme of Henry, Tang and Heinecke,
// "Leveraging the bfloat16 Artificial Intelligence Datatype For
// Higher-Precision Computations" (ARITH 2019), here on gfx950's bf16 MFMA.
//
// Layout as in gemm_f32.h (one 256-thread workgroup per T x T output tile,
// 4 waves in a 2 x 2 grid of (T/2) x (T/2) sub-tiles, 32 k-values per chunk,
// the MFMA result layout is the same), except that each operand is staged as
// three bf16 planes [3][T][XS] with k contiguous: a 16-byte LDS read gives a
// lane its 8 consecutive k-values of one row, which is the bf16 MFMA operand.
// The split happens when a chunk goes from registers to LDS.  One LDS buffer
// (so that two workgroups fit on a CU): the next chunk's global loads are in
// flight while the current chunk is multiplied, then written after a barrier.
#pragma once

#include "gemm_f32.h"

namespace sg {

typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

constexpr int XS = GBK + 8;  // LDS row stride in bf16 (80 bytes: conflict-free 16-byte reads)

template <int T>
struct X6Lds {
  static constexpr int PLANE = T * XS;                 // bf16 per plane
  static constexpr int OPER = 3 * PLANE;               // bf16 per operand
  static constexpr int BYTES = 2 * OPER * 2;           // both operands
  static constexpr int EPI = T * (T + 4) * 4;          // epilogue staging (fp32)
  static constexpr int SIZE = BYTES > EPI ? BYTES : EPI;
  static constexpr int SHORT = 2 * BYTES > EPI ? 2 * BYTES : EPI;  // two chunk buffers
};

typedef float floatx2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// (a, b) -> their h, m and l parts as packed bf16 pairs (a in the low half):
// one round-to-nearest-even pair conversion per part; the value of a packed
// bf16 is its bits moved to the top of an fp32 word.
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& hp, uint32_t& mp, uint32_t& lp) {
  hp = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2v){a, b}, bf16x2v));
  const float ra = a - __uint_as_float(hp << 16), rb = b - __uint_as_float(hp & 0xffff0000u);
  mp = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2v){ra, rb}, bf16x2v));
  const float sa = ra - __uint_as_float(mp << 16), sb = rb - __uint_as_float(mp & 0xffff0000u);
  lp = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2v){sa, sb}, bf16x2v));
}

// four values split and written to the three planes (8 bytes each)
__device__ __forceinline__ void store_split4(__bf16* lds, int plane, int off, const floatx4& x) {
  uint32_t h0, m0, l0, h1, m1, l1;
  split3_pair(x[0], x[1], h0, m0, l0);
  split3_pair(x[2], x[3], h1, m1, l1);
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2v*>(lds + 0 * plane + off) = u32x2v{h0, h1};
  *reinterpret_cast<u32x2v*>(lds + 1 * plane + off) = u32x2v{m0, m1};
  *reinterpret_cast<u32x2v*>(lds + 2 * plane + off) = u32x2v{l0, l1};
}

// Rows of a k-contiguous fp32 matrix with 16-byte aligned rows (as
// RowsF32VT): element (r, k) = src[r*ld + k], valid for r < rows, k < kend
// (kend % 4 == 0); stored split into the three planes.  A chunk with every
// row present and every k below kend is read from a workgroup-uniform base
// plus a 32-bit per-lane offset (no per-element address arithmetic); other
// chunks use clamped addresses and zero what lies outside.  FULL: the caller
// guarantees rows == T, kend a multiple of 32 and ld < 2^24 (only the first
// path is compiled).
template <int T, bool FULL = false>
struct RowsX6V {
  const float* src;
  int64_t ld;
  int rows;
  int64_t kend;
  floatx4 v[T / 32];
  __device__ inline void load(int64_t k0) {
    const int k4 = (threadIdx.x & 7) * 4, r0 = threadIdx.x >> 3;
    if (FULL || (rows == T && k0 + GBK <= kend && ld < (int64_t(1) << 24))) {
      const uint32_t voff = (uint32_t)(r0 * ld + k4) * 4u;
#pragma unroll
      for (int u = 0; u < T / 32; ++u) {
        const char* base = reinterpret_cast<const char*>(src + 32 * u * ld + k0);
        v[u] = *reinterpret_cast<const floatx4*>(base + voff);
      }
      return;
    }
    const int64_t k = k0 + k4;
    const int64_t kc = k < kend ? k : kend - 4;
#pragma unroll
    for (int u = 0; u < T / 32; ++u) {
      const int r = r0 + 32 * u;
      const int rc = r < rows ? r : rows - 1;
      v[u] = *reinterpret_cast<const floatx4*>(src + (int64_t)rc * ld + kc);
    }
  }
  __device__ inline void store(__bf16* lds, int64_t k0) {
    const int k4 = (threadIdx.x & 7) * 4, r0 = threadIdx.x >> 3;
    const bool kok = FULL || k0 + k4 < kend;
#pragma unroll
    for (int u = 0; u < T / 32; ++u) {
      const int r = r0 + 32 * u;
      const floatx4 x = (FULL || (r < rows && kok)) ? v[u] : floatx4{0.f, 0.f, 0.f, 0.f};
      store_split4(lds, X6Lds<T>::PLANE, r * XS + k4, x);
    }
  }
};

// Row-major [k][j] fp32 read transposed (as ColsF32TT): thread t owns column
// j = t % T and KT = 32 T / 256 consecutive k; element (j, k) = src[k*ld + j],
// valid for j < cols, k < kend; stored split into the three planes.  The k
// range of a thread is the same for its whole wave, so a full chunk is read
// from uniform row addresses plus the lane's column offset.  FULL: the caller
// guarantees cols == T and kend a multiple of 32.
template <int T, bool FULL = false>
struct ColsX6T {
  static constexpr int KT = GBK * T / GTHREADS;  // 16 (T = 128) or 8 (T = 64)
  const float* src;
  int64_t ld;
  int cols;
  int64_t kend;
  float v[KT];
  __device__ inline void load(int64_t k0) {
    const int j = threadIdx.x % T;
    const int kb = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / T)) * KT;
    if (FULL || (cols == T && k0 + GBK <= kend)) {
      const uint32_t voff = (uint32_t)j * 4u;
#pragma unroll
      for (int u = 0; u < KT; ++u) {
        const char* base = reinterpret_cast<const char*>(src + (k0 + kb + u) * ld);
        v[u] = *reinterpret_cast<const float*>(base + voff);
      }
      return;
    }
    const int jc = j < cols ? j : cols - 1;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      const int64_t k = k0 + kb + u;
      const int64_t kc = k < kend ? k : kend - 1;
      v[u] = src[kc * ld + jc];
    }
  }
  __device__ inline void store(__bf16* lds, int64_t k0) {
    const int j = threadIdx.x % T, kb = (threadIdx.x / T) * KT;
#pragma unroll
    for (int q = 0; q < KT / 4; ++q) {
      floatx4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (FULL || (j < cols && k0 + kb + 4 * q + e < kend)) ? v[4 * q + e] : 0.f;
      store_split4(lds, X6Lds<T>::PLANE, j * XS + kb + 4 * q, x);
    }
  }
};

// acc += P[0:T, 0:32] * Q[0:T, 0:32]^T from the split planes in LDS.  The Q
// fragments are read once; the P fragments one row block at a time.
template <int T>
__device__ inline void tile_mma_x6(TileAccT<T>& acc, const __bf16* Pl, const __bf16* Ql, int wave, int lane) {
  constexpr int NI = T / 32;
  constexpr int PL = X6Lds<T>::PLANE;
  const int prow = (wave >> 1) * (T / 2) + (lane & 15);
  const int qrow = (wave & 1) * (T / 2) + (lane & 15);
  const int k = (lane >> 4) * 8;
  bf16x8v q[NI][3];
#pragma unroll
  for (int j = 0; j < NI; ++j)
#pragma unroll
    for (int s = 0; s < 3; ++s) q[j][s] = *reinterpret_cast<const bf16x8v*>(Ql + s * PL + (qrow + j * 16) * XS + k);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    bf16x8v p[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) p[s] = *reinterpret_cast<const bf16x8v*>(Pl + s * PL + (prow + i * 16) * XS + k);
    // smallest terms first
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      floatx4 a = acc.v[i][j];
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p[1], q[j][1], a, 0, 0, 0);  // mm
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p[0], q[j][2], a, 0, 0, 0);  // hl
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p[2], q[j][0], a, 0, 0, 0);  // lh
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p[0], q[j][1], a, 0, 0, 0);  // hm
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p[1], q[j][0], a, 0, 0, 0);  // mh
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p[0], q[j][0], a, 0, 0, 0);  // hh
      acc.v[i][j] = a;
    }
  }
}

// acc += P * Q^T over k in [0, K); lds holds X6Lds<T>::SIZE bytes.  With
// DEPTH = 2 the global loads run two chunks ahead (two register sets): a
// chunk's products take less time than a load's round trip under load.
// DEPTH = 1 loads one chunk ahead (fewer registers).
template <int T, int DEPTH = 2, class PL, class QL>
__device__ inline void tile_gemm_x6(TileAccT<T>& acc, PL& pl, QL& ql, int64_t K, void* lds) {
  __bf16* Pl = static_cast<__bf16*>(lds);
  __bf16* Ql = Pl + X6Lds<T>::OPER;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nch = ceil_div(K, GBK);
  if (nch <= 0) return;
  if constexpr (DEPTH == 1) {
    pl.load(0);
    ql.load(0);
    pl.store(Pl, 0);
    ql.store(Ql, 0);
    __syncthreads();
    for (int64_t c = 0; c < nch; ++c) {
      const bool more = c + 1 < nch;
      if (more) {
        pl.load((c + 1) * GBK);
        ql.load((c + 1) * GBK);
      }
      tile_mma_x6(acc, Pl, Ql, wave, lane);
      if (more) {
        __syncthreads();
        pl.store(Pl, (c + 1) * GBK);
        ql.store(Ql, (c + 1) * GBK);
        __syncthreads();
      }
    }
    return;
  }
  PL pl2 = pl;
  QL ql2 = ql;
  pl.load(0);
  ql.load(0);
  if (nch > 1) {
    pl2.load(GBK);
    ql2.load(GBK);
  }
  pl.store(Pl, 0);
  ql.store(Ql, 0);
  __syncthreads();
  for (int64_t c = 0; c < nch; c += 2) {
    // chunk c is in LDS, chunk c+1 in (pl2, ql2); (pl, ql) takes chunk c+2
    if (c + 2 < nch) {
      pl.load((c + 2) * GBK);
      ql.load((c + 2) * GBK);
    }
    tile_mma_x6(acc, Pl, Ql, wave, lane);
    if (c + 1 >= nch) break;
    __syncthreads();
    pl2.store(Pl, (c + 1) * GBK);
    ql2.store(Ql, (c + 1) * GBK);
    __syncthreads();
    // chunk c+1 is in LDS, chunk c+2 in (pl, ql); (pl2, ql2) takes chunk c+3
    if (c + 3 < nch) {
      pl2.load((c + 3) * GBK);
      ql2.load((c + 3) * GBK);
    }
    tile_mma_x6(acc, Pl, Ql, wave, lane);
    if (c + 2 >= nch) break;
    __syncthreads();
    pl.store(Pl, (c + 2) * GBK);
    ql.store(Ql, (c + 2) * GBK);
    __syncthreads();
  }
}

// acc += P * Q^T for K <= 32 NCH, every operand load issued up front: the
// short contractions (one block of errors, one panel) are latency bound, and
// this takes one global round trip instead of one per chunk.  Two LDS
// buffers, one barrier per chunk; lds holds X6Lds<T>::SHORT bytes.
template <int T, int NCH, class PL, class QL>
__device__ inline void tile_gemm_x6_short(TileAccT<T>& acc, const PL& pl0, const QL& ql0, int64_t K,
                                          void* lds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = (int)ceil_div(K, GBK);
  PL pl[NCH];
  QL ql[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    pl[c] = pl0;
    ql[c] = ql0;
    if (c < nch) {
      pl[c].load(c * GBK);
      ql[c].load(c * GBK);
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c >= nch) break;
    __bf16* Pl = static_cast<__bf16*>(lds) + (c & 1) * 2 * X6Lds<T>::OPER;
    __bf16* Ql = Pl + X6Lds<T>::OPER;
    pl[c].store(Pl, c * GBK);
    ql[c].store(Ql, c * GBK);
    __syncthreads();
    tile_mma_x6(acc, Pl, Ql, wave, lane);
  }
}

}  // namespace sg
