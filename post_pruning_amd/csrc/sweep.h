// Column sweep kernels of the SparseGPT layer solver, shared by the
// translation units that instantiate them (plain, quantized and vector-level
// variants compile in parallel) and by the host code of the prune call.
#pragma once

#include "gemm_f32.h"

#include <math.h>

#include <type_traits>
#include <utility>

namespace sg {

constexpr int SB = SG_MAX_BLOCKSIZE;  // 128
constexpr int EGK = 512;              // columns of a lazy-update group (error buffer width)

enum { MODE_THRESH = 0, MODE_NM = 1, MODE_FORCED = 2, MODE_ROW = 3 };

// Radix-select buffers, double-buffered by block parity: the sweep of block b
// clears the set block b + 1 will use while nobody reads it.
struct SelSet {
  unsigned hist0[kSelBins];   // top 11 bits of every key
  unsigned hist1[kSelBins];   // next 11 bits of the keys under the top digit
  unsigned ncand;             // keys gathered under the top digit
  unsigned pad[63];
};
struct SelState {
  SelSet set[2];
};

// Row segments of one prune call (kernel argument): segment p is rows
// [row0[p], row0[p+1]) with the factor U[p]; its sweep workgroups are
// [wg0[p], wg0[p+1]) (16 times the rows per lane, 32 or 64 rows each); k[p]
// keys of each block are pruned under block-global selection (fixed[p]: 2
// none, 3 all, 0 selected by the radix passes).
struct Segs {
  int n;
  int64_t row0[SG_MAX_SEGMENTS + 1];
  int wg0[SG_MAX_SEGMENTS + 1];
  long long k[SG_MAX_SEGMENTS];
  int fixed[SG_MAX_SEGMENTS];
  const float* U[SG_MAX_SEGMENTS];
};

// OBS saliency w^2 / U_cc^2 as (w * rd)^2 with rd = 1 / U_cc (the IEEE
// quotient, formed the same way wherever a saliency is taken, so that every
// kernel ranks the same fp32 values).
__device__ inline float saliency(float w, float rd) {
  const float q = w * rd;
  return q * q;
}

__device__ inline unsigned long long sal_key(float w, float rd, uint32_t lin) {
  return ((unsigned long long)__float_as_uint(saliency(w, rd)) << 32) | lin;
}

__device__ inline void sel_clear_set(SelSet& s, int tid, int nthreads) {
  for (int b = tid; b < kSelBins; b += nthreads) {
    s.hist0[b] = 0u;
    s.hist1[b] = 0u;
  }
  if (tid == 0) s.ncand = 0u;
}

// Exact k-th smallest 64-bit key (bits(W^2 / U_cc^2) << 32 | r*n + c) of the
// m x w block, radix select with 11-bit digits, saliency bits first:
//   pass 0  every workgroup histograms the top digit of its keys (eight
//           lane-interleaved LDS sub-histograms against contention on hot
//           bins) and adds it into the block's global histogram;
//   pass 1  every workgroup scans that histogram itself (2048 bins), fixes the
//           top digit, histograms the next digit of the keys under it and
//           gathers those keys into a candidate list;
//   sweep   every sweep workgroup scans the second histogram, fixes the second
//           digit, and either takes the whole bucket or sorts the keys under
//           both digits (gathered from the candidate list) in LDS and reads
//           off the one of the remaining rank.
// No workgroup waits for another: each kernel consumes what the previous one
// completed.
constexpr int SEL_KPT = 16;    // keys per thread
constexpr int SEL_SUB = 8;     // LDS sub-histograms
constexpr int SEL_SORT = 8192; // keys sorted in LDS

// Scan of a 2048-bin histogram (256 threads, thread t owns bins 8t..8t+7):
// the bin holding the krem-th key, the keys before it and its count, in LDS.
struct HistPick {
  unsigned digit, cnt;
  unsigned long long before;
  unsigned wsum[4];
};

__device__ inline void hist_locate(const unsigned* hist, long long krem, HistPick& P) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int per = kSelBins / 256;
  unsigned cnt[per];
  unsigned local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    cnt[i] = hist[tid * per + i];
    local += cnt[i];
  }
  unsigned incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) P.wsum[wave] = incl;
  __syncthreads();
  unsigned wbase = 0;
  for (int wv = 0; wv < wave; ++wv) wbase += P.wsum[wv];
  unsigned long long cum = (unsigned long long)(wbase + incl - local);
  const unsigned long long after = (unsigned long long)(wbase + incl);
  if ((long long)cum < krem && krem <= (long long)after) {
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const unsigned cn = cnt[i];
      if ((long long)cum < krem && (long long)(cum + cn) >= krem) {
        P.digit = (unsigned)(tid * per + i);
        P.before = cum;
        P.cnt = cn;
      }
      cum += cn;
    }
  }
  __syncthreads();
}

// Threshold key of the block from the two histograms and the candidates
// (run by every sweep workgroup; `scratch` holds SEL_SORT keys of LDS).
__device__ __forceinline__ unsigned long long select_finish(const SelSet& ss, const unsigned long long* cand,
                                            long long k, unsigned long long* scratch,
                                            unsigned* s_cnt, HistPick& P) {
  const int tid = threadIdx.x;
  hist_locate(ss.hist0, k, P);
  const unsigned d0 = P.digit;
  const long long k1 = k - (long long)P.before;
  hist_locate(ss.hist1, k1, P);
  const unsigned long long pf = ((unsigned long long)d0 << 53) | ((unsigned long long)P.digit << 42);
  long long kr = k1 - (long long)P.before;
  const unsigned cnt = P.cnt;
  if ((long long)cnt == kr) return pf | ((1ull << 42) - 1ull);  // the bucket is taken whole
  const unsigned ncand = ss.ncand;
  const unsigned long long fmask2 = ~((1ull << 42) - 1ull);
  if (cnt <= (unsigned)SEL_SORT) {
    if (tid == 0) *s_cnt = 0u;
    __syncthreads();
    // candidates read 16 per thread at a time, all loads in flight together
    for (unsigned base = 0; base < ncand; base += 256 * 16) {
      unsigned long long kv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const unsigned i = base + u * 256 + tid;
        kv[u] = cand[i < ncand ? i : ncand - 1];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const unsigned i = base + u * 256 + tid;
        if (i < ncand && (kv[u] & fmask2) == pf) scratch[atomicAdd(s_cnt, 1u)] = kv[u];
      }
    }
    __syncthreads();
    const unsigned got = *s_cnt;
    unsigned sz = 1;
    while (sz < got) sz <<= 1;
    for (unsigned i = got + tid; i < sz; i += 256) scratch[i] = ~0ull;
    __syncthreads();
    for (unsigned kk = 2; kk <= sz; kk <<= 1) {
      for (unsigned j = kk >> 1; j > 0; j >>= 1) {
        for (unsigned i = tid; i < sz; i += 256) {
          const unsigned ixj = i ^ j;
          if (ixj > i) {
            const unsigned long long a = scratch[i], b = scratch[ixj];
            if ((a > b) == ((i & kk) == 0)) {
              scratch[i] = b;
              scratch[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    const unsigned long long t = scratch[kr - 1];
    __syncthreads();
    return t;
  }
  // too many keys under both digits to sort: radix passes over the list,
  // with the first 2048 words of scratch as the histogram
  unsigned* h = reinterpret_cast<unsigned*>(scratch);
  unsigned long long p2 = pf;
  static constexpr int kShift[4] = {32, 21, 10, 0};
  static constexpr int kWidth[4] = {10, 11, 11, 10};
  for (int p = 0; p < 4; ++p) {
    const int sh = kShift[p];
    const unsigned dm = (1u << kWidth[p]) - 1u;
    const unsigned long long fm = ~((1ull << (sh + kWidth[p])) - 1ull);
    for (int b = tid; b < kSelBins; b += 256) h[b] = 0u;
    __syncthreads();
    for (unsigned base = 0; base < ncand; base += 256 * 16) {
      unsigned long long kv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const unsigned i = base + u * 256 + tid;
        kv[u] = cand[i < ncand ? i : ncand - 1];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const unsigned i = base + u * 256 + tid;
        if (i < ncand && (kv[u] & fm) == p2) atomicAdd(&h[(unsigned)(kv[u] >> sh) & dm], 1u);
      }
    }
    __syncthreads();
    hist_locate(h, kr, P);
    p2 |= (unsigned long long)P.digit << sh;
    kr -= (long long)P.before;
    if ((long long)P.cnt == kr || sh == 0) {
      const unsigned long long t = p2 | ((sh > 0) ? ((1ull << sh) - 1ull) : 0ull);
      __syncthreads();
      return t;
    }
    __syncthreads();
  }
  return ~0ull;  // not reached
}

// ---- in-block sweep ---------------------------------------------------------
// One wave per 16 rows (8 with two rows per lane, RPL below); the block's
// columns are held in registers as eight 16x16 tiles in the fp32 MFMA
// accumulator layout (lane l, register v: row 4*(l/16) + v, column l%16 of
// the tile).  Per 16-column chunk c:
//   * the 16 columns are swept in order: the owner lanes (column j of the
//     chunk) compute e = W[r,J] / U_JJ for pruned entries, a DPP row
//     broadcast hands e to the other 15 lanes of the row, which subtract
//     e * U[J, col] (U is zero left of the diagonal, so earlier columns are
//     untouched);
//   * the chunk's errors E_c (16 x 16) then update every later chunk,
//     W[:, c'] -= E_c U[c, c'], on v_mfma_f32_16x16x4_f32 (E_c goes through a
//     small per-wave LDS tile to reach the A-operand layout): chunk c + 1 at
//     once, the chunks after it during chunk c + 1's column steps.
// This is the same computation as the column-by-column OBS sweep, with the
// updates of later chunks batched (they only add into columns not yet
// reached).  The U block (upper triangle, zero elsewhere) sits in LDS.
// Template variants of one kernel: MODE (block-global threshold, N:M,
// per-row, forced mask), MGS (N:M groups of up to 16 columns, ranked inside
// the column steps), QUANT (kept weights rounded to their row's grid at their
// step) and JOINT (each 16-column chunk's chosen weights removed together).
constexpr int SWS = SB + 4;  // LDS row stride of the U block (floats)
constexpr int ESS = 20;      // per-wave E tile row stride (floats)

constexpr int GCS = 17;      // row stride of a chunk's 16 x 16 Gram matrix

struct SweepLds {
  float Ub[SB * SWS];
  float Rd[SB];          // 1 / U_JJ (0 past the block)
  float Es[4][16 * ESS];
  float Tw[4][16 * SWS]; // per-wave 16 x 128 staging tile (row-major), N:M scratch
  float Gc[8][16 * GCS]; // vector-level mode: Gram U16^T U16 of each chunk's diagonal block
};

// Lane L of every 16-lane row to the whole row (DPP row_newbcast).
template <int L>
__device__ inline float bcast16_c(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + L, 0xF, 0xF, true));
}

// lexicographic (saliency, position) rank among cnt values
__device__ __forceinline__ int rank_of(const float* sal, int cnt, float my, int me) {
  int rank = 0;
  for (int t = 0; t < cnt; ++t) {
    const float o = sal[t];
    rank += (o < my || (o == my && t < me)) ? 1 : 0;
  }
  return rank;
}

// Sum of x over the 16 lanes of a DPP row, returned in every lane of the row
// (Hillis-Steele scan by row_shr 1, 2, 4, 8, then lane 15 broadcast).
__device__ __forceinline__ int rowsum16(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, 0x118, 0xF, 0xF, true);
  return __builtin_amdgcn_mov_dpp(x, 0x15F, 0xF, 0xF, true);
}

// Per-chunk constants of one lane (its column col = 16c + lc of the chunk):
//   g[j] = U[16c + j][col] / U_JJ for j != lc, 0 for j == lc;
// the owner lane of column J keeps its value frozen from step J on, so the
// chunk's errors can be formed at its end from the registers.
struct ChunkCtx {
  float g[16];
  float rd;      // 1 / U_col,col
  float ucc;     // U_col,col
};

// Grid of the joint sparse + quantized sweep for the lane's four rows:
// value = s * (code - z), code = clamp(round(x / s) + z, 0, L), rounding half
// to even (x / s taken as x * (1 / s)).
struct RowQuant {
  float s[4], inv[4], z[4];
  float L;
};

__device__ __forceinline__ float quant_value(float x, const RowQuant& q, int v) {
  const float c = fminf(fmaxf(rintf(x * q.inv[v]) + q.z[v], 0.f), q.L);
  return q.s[v] * (c - q.z[v]);
}

// N:M ranking of the group of MGS columns at lanes J .. J+MGS-1 of each
// 16-lane row.  A saliency is nonnegative, so its fp32 bit pattern orders as
// its value does: the (saliency, position) order is an unsigned compare of the
// bits, against the lane's own bits plus one for members at earlier positions
// (equal saliency, earlier column: ahead).  Member T's bits reach every lane
// of the row by a DPP broadcast; no branch, so the four rows interleave.
template <int J, int T>
__device__ __forceinline__ unsigned ahead_u(unsigned my, unsigned my1, int lc) {
  const unsigned o = (unsigned)__builtin_amdgcn_mov_dpp((int)my, 0x150 + J + T, 0xF, 0xF, true);
  return o < (lc > J + T ? my1 : my) ? 1u : 0u;
}

template <int J, int... Ts>
__device__ __forceinline__ unsigned group_rank_u(std::integer_sequence<int, Ts...>, unsigned my, int lc) {
  const unsigned my1 = my + 1u;
  return (ahead_u<J, Ts>(my, my1, lc) + ... + 0u);
}

// Bits v = 0..RPL-1 (the lane's rows): the lane's column is in the group and
// ranks among its MGS - nkeep smallest, so it is pruned.
template <int J, int MGS, int RPL = 4>
__device__ __forceinline__ unsigned group_pruned(const floatx4& Wc, float rd, int lc, int nkeep,
                                                 unsigned rowbits) {
  const unsigned lim = (unsigned)(MGS - nkeep);
  unsigned bits = 0u;
#pragma unroll
  for (int v = 0; v < RPL; ++v) {
    const unsigned my = __float_as_uint(saliency(Wc[v], rd));
    const unsigned rank = group_rank_u<J>(std::make_integer_sequence<int, MGS>{}, my, lc);
    bits |= (rank < lim ? 1u : 0u) << v;
  }
  const bool in = lc >= J && lc < J + MGS;
  return in ? bits & rowbits : 0u;
}

// ---- vector-level (joint) removal of one 16-column chunk -------------------
// Every row removes its chosen columns P of the chunk at once: with the
// chunk's Gram G = U16^T U16 (U16 = the chunk's diagonal 16 x 16 block of U,
// so G_PP is the inverse Hessian of the free columns restricted to P) it
// solves G_PP y = w_P and takes the error row e = U16 y (e_J = sum_i
// U16[J][i] y_i), which moves the row by -e U: its chosen weights land on 0
// and every free weight takes the least-squares adjustment.  The system is
// kept 16 x 16 for every row (identity on the kept columns, right-hand side
// 0 there).  Lane j of a 16-lane row owns column j: a right-looking Cholesky
// with DPP row broadcasts of the pivot and of each lane's multiplier, then
// forward and backward substitution.
template <int S, int I>
__device__ __forceinline__ void chol_upd1(float (&a)[16], float lv, float lvm) {
  if constexpr (I > S) a[I] = fmaf(-bcast16_c<I>(lv), lvm, a[I]);
}

template <int S, int... Is>
__device__ __forceinline__ void chol_update(std::integer_sequence<int, Is...>, float (&a)[16], float lv,
                                            float lvm) {
  (chol_upd1<S, Is>(a, lv, lvm), ...);
}

// step S: pivot a_SS from lane S; lanes j > S update their column; lane j
// keeps l_jS (its row of L) and, at S == j, 1 / l_jj
template <int S>
__device__ __forceinline__ void chol_step(float (&a)[16], float (&lrow)[16], float& rj, int lc) {
  const float r = __builtin_amdgcn_rsqf(bcast16_c<S>(a[S]));
  const float lv = a[S] * r;
  lrow[S] = lv;
  rj = lc == S ? r : rj;
  chol_update<S>(std::make_integer_sequence<int, 16>{}, a, lv, lc > S ? lv : 0.f);
}

template <int S>
__device__ __forceinline__ void fwd_step(float& bp, const float (&lrow)[16], float rj, int lc) {
  const float zs = bcast16_c<S>(bp * rj);
  bp = lc > S ? fmaf(-lrow[S], zs, bp) : bp;
}

template <int S>
__device__ __forceinline__ void bwd_step(float& acc, const float (&a)[16], float z, float rj, int lc, float& e,
                                         float urow) {
  const float ys = bcast16_c<S>((z - rj * acc) * rj);
  acc = lc < S ? fmaf(a[S], ys, acc) : acc;
  e = fmaf(urow, ys, e);
}

template <int... Ss>
__device__ __forceinline__ void joint_solve(std::integer_sequence<int, Ss...>, float (&a)[16], float bp,
                                            const float (&urow)[16], int lc, float& e) {
  float lrow[16];
  float rj = 1.f;
  (chol_step<Ss>(a, lrow, rj, lc), ...);
  (fwd_step<Ss>(bp, lrow, rj, lc), ...);
  const float z = bp * rj;
  float acc = 0.f;
  e = 0.f;
  (bwd_step<15 - Ss>(acc, a, z, rj, lc, e, urow[15 - Ss]), ...);
}

template <int J, int MGS, int RPL>
__device__ __forceinline__ void rank_step(const floatx4& Wc, unsigned& Pc, const ChunkCtx& cx, int lc,
                                          int nkeep, unsigned rowbits) {
  if constexpr (MGS > 0) {
    if constexpr ((J % MGS) == 0) Pc |= group_pruned<J, MGS, RPL>(Wc, cx.rd, lc, nkeep, rowbits);
  }
}

template <int J, int RPL>
__device__ __forceinline__ void apply_step(floatx4& Wc, const float (&d)[4], const ChunkCtx& cx) {
  float e[4];
#pragma unroll
  for (int v = 0; v < RPL; ++v) e[v] = bcast16_c<J>(d[v]);
#pragma unroll
  for (int v = 0; v < RPL; ++v) Wc[v] = fmaf(-e[v], cx.g[J], Wc[v]);
}

// The chunk's vector-level step: groups of M <= 16 ranked at the chunk start,
// then the joint solve per row, then the chunk's own columns moved by -e U16
// (the owner lane's own term is taken at the chunk end).  Returns e per row.
template <int MGS, int RPL, int... Js>
__device__ __forceinline__ void joint_chunk(std::integer_sequence<int, Js...> seq, floatx4& Wc, unsigned& Pc,
                                            const ChunkCtx& cx, int lc, int lg, int nkeep, unsigned rowbits,
                                            const float* Gc, const float* Urow, float (&ev)[4]) {
  (rank_step<Js, MGS, RPL>(Wc, Pc, cx, lc, nkeep, rowbits), ...);
  float gcol[16], urow[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    gcol[i] = Gc[i * GCS + lc];
    urow[i] = Urow[i];
  }
  // the lane's rows one after another (one copy of the solve in the code)
#pragma unroll 1
  for (int v = 0; v < RPL; ++v) {
    const float wv = v == 0 ? Wc[0] : (v == 1 ? Wc[1] : (v == 2 ? Wc[2] : Wc[3]));
    const unsigned long long bal = __ballot((Pc >> v) & 1u);
    const unsigned rowP = (unsigned)(bal >> (16 * lg)) & 0xFFFFu;
    const bool mine = (rowP >> lc) & 1u;
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = (mine && ((rowP >> i) & 1u)) ? gcol[i] : (i == lc ? 1.f : 0.f);
    float e;
    joint_solve(seq, a, mine ? wv : 0.f, urow, lc, e);
    ev[0] = v == 0 ? e : ev[0];
    ev[1] = v == 1 ? e : ev[1];
    ev[2] = v == 2 ? e : ev[2];
    ev[3] = v == 3 ? e : ev[3];
  }
  float d[4];
#pragma unroll
  for (int v = 0; v < RPL; ++v) d[v] = ev[v] * cx.ucc;
  (apply_step<Js, RPL>(Wc, d, cx), ...);
}

// Sweep column J of the chunk (compile-time J: static DPP lane and indices).
// Chain per step and row: select (pruned ? W_J : 0) on the owner lane, DPP
// broadcast over the 16 lanes of the row, fused multiply-add.
template <int J, int MGS, bool QUANT, int RPL>
__device__ __forceinline__ void sweep_step(floatx4& Wc, unsigned& Pc, const ChunkCtx& cx, int lc,
                                           int nkeep, unsigned rowbits, const RowQuant& q) {
  if constexpr (MGS > 0) {
    if constexpr ((J % MGS) == 0) {
      // N:M group of MGS <= 16 columns = lanes J .. J+MGS-1 of the row,
      // ranked from the current saliencies at the group start
      Pc |= group_pruned<J, MGS, RPL>(Wc, cx.rd, lc, nkeep, rowbits);
    }
  }
  // owner lane's deviation from its target (0 if pruned, the grid value if
  // kept and quantized), times U_JJ: the DPP broadcast hands it to the row
  float e[4];
#pragma unroll
  for (int v = 0; v < RPL; ++v) {
    float d;
    if constexpr (QUANT)
      d = ((Pc >> v) & 1u) ? Wc[v] : Wc[v] - quant_value(Wc[v], q, v);
    else
      d = ((Pc >> v) & 1u) ? Wc[v] : 0.f;
    e[v] = bcast16_c<J>(d);
  }
#pragma unroll
  for (int v = 0; v < RPL; ++v) Wc[v] = fmaf(-e[v], cx.g[J], Wc[v]);
}

template <int MGS, bool QUANT, int RPL, int... Js>
__device__ __forceinline__ void sweep_chunk(std::integer_sequence<int, Js...>, floatx4& Wc, unsigned& Pc,
                                            const ChunkCtx& cx, int lc, int nkeep, unsigned rowbits,
                                            const RowQuant& q) {
  (sweep_step<Js, MGS, QUANT, RPL>(Wc, Pc, cx, lc, nkeep, rowbits, q), ...);
}

// RPL: rows per lane, 4 (16 rows a wave, 64 a workgroup) or 2 (8 and 32:
// twice the workgroups, half the column-step work a SIMD, for layers whose
// rows then still fit one workgroup per CU).  A lane's rows sit at positions
// 4 lg + v (v < RPL) of the 16-row MFMA tiles; with RPL = 2 the other two
// positions are idle rows of zeros.
template <int MODE, int MGS, bool QUANT, bool JOINT = false, int RPL = 4>
__global__ __launch_bounds__(256) void sweep_kernel(float* __restrict__ W, uint8_t* __restrict__ mask_out,
                                                    float* __restrict__ Err,
                                                    const uint8_t* __restrict__ mask_in,
                                                    SelState* __restrict__ st,
                                                    const unsigned long long* __restrict__ cand,
                                                    int parity, const Segs segs,
                                                    int64_t n, int64_t i1, int w, int nkeep,
                                                    int mgroup, uint8_t* __restrict__ codes_out,
                                                    const float* __restrict__ qscale,
                                                    const float* __restrict__ qzero, float qlevels) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SweepLds& S = *reinterpret_cast<SweepLds*>(smem);
  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: held in a scalar register
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lc = lane & 15;       // column inside a chunk
  const int lg = lane >> 4;       // row group: rows RPL*lg .. RPL*lg+RPL-1 of the wave's
  constexpr int RW = 4 * RPL;     // rows of a wave
  // this workgroup's segment (matrix): its rows end at m
  int seg = 0;
  while (seg + 1 < segs.n && (int)blockIdx.x >= segs.wg0[seg + 1]) ++seg;
  const int64_t m = segs.row0[seg + 1];
  const float* __restrict__ U = segs.U[seg];
  const int64_t rbase = segs.row0[seg] + ((int64_t)blockIdx.x - segs.wg0[seg]) * (4 * RW);
  const long long ksel = segs.k[seg];
  const int sel_fixed = segs.fixed[seg];
  SelState* const stp = st + seg;
  const unsigned long long* const candp = cand + segs.row0[seg] * SB;
  const int64_t r0 = rbase + wave * RW + RPL * lg;
  const int nch = (w + 15) >> 4;
  RowQuant q;
  if constexpr (QUANT) {
#pragma unroll
    for (int v = 0; v < RPL; ++v) {
      const int64_t r = r0 + v < m ? r0 + v : m - 1;
      q.s[v] = qscale[r];
      q.inv[v] = 1.f / q.s[v];
      q.z[v] = qzero[r];
    }
    q.L = qlevels;
  }

  // Every global load of the block is issued before anything waits on one:
  // the U block (16-byte loads, pass u covers rows 8u .. 8u+7, one wave
  // instruction reads two whole 512-byte rows; clamped in-bounds addresses,
  // rows/columns past the block re-read the last one), its diagonal, the
  // wave's W tile and, for a forced mask, its mask bytes.  Their latencies
  // overlap each other and the threshold search.
  const bool uvec = ((n & 3) == 0) && ((i1 & 3) == 0);  // 16-byte aligned rows
  floatx4 uv[16];
  if (uvec && w == SB && n < (int64_t(1) << 24)) {
    // full block: pass u reads rows 8u + tid/32 from a uniform base (row
    // i1 + 8u) plus the thread's 32-bit offset
    const uint32_t uoff = (uint32_t)((tid >> 5) * n + (tid & 31) * 4) * 4u;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const char* base = reinterpret_cast<const char*>(U + (i1 + 8 * u) * n + i1);
      uv[u] = *reinterpret_cast<const floatx4*>(base + uoff);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int f = u * 256 + tid;
      const int j = f >> 5, c4 = (f & 31) * 4;
      const int jc = j < w ? j : w - 1;
      const float* urow = U + (i1 + jc) * n + i1;
      if (uvec && c4 + 4 <= w) {
        uv[u] = *reinterpret_cast<const floatx4*>(urow + c4);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) uv[u][e] = urow[c4 + e < w ? c4 + e : w - 1];
      }
    }
  }
  const int dj = tid < w ? tid : w - 1;
  const float udiag = U[(i1 + dj) * n + i1 + dj];

  // Block columns in registers; rows past m read row m-1 and stay unwritten.
  // With 16-byte aligned rows the tile goes through the wave's LDS staging
  // area: coalesced 16-byte global accesses (one wave instruction = two
  // 512-byte rows), accumulator layout on the LDS side.
  const bool vio = ((n & 3) == 0) && ((i1 & 3) == 0) && ((w & 3) == 0) &&
                   ((reinterpret_cast<uintptr_t>(W) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(mask_in) & 3) == 0) &&
                   ((reinterpret_cast<uintptr_t>(mask_out) & 3) == 0) &&
                   ((reinterpret_cast<uintptr_t>(codes_out) & 3) == 0) &&
                   ((reinterpret_cast<uintptr_t>(Err) & 15) == 0);
  float* Tw = S.Tw[wave];
  const int64_t rw0 = rbase + wave * RW;
  bool rowok[4];
  floatx4 Wt[8], Et[8];
  unsigned Pm[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) rowok[v] = v < RPL && r0 + v < m;
  // the wave's RW x 128 tile in RW / 2 passes of two 512-byte rows
  constexpr int WP = RW / 2;
  floatx4 wt[WP];
  unsigned mw[WP];
  if (vio && w == SB && rw0 + RW <= m && n < (int64_t(1) << 24)) {
    // full tile: pass u reads rows 2u + lane/32 from a uniform base
    const uint32_t woff = (uint32_t)((lane >> 5) * n + (lane & 31) * 4) * 4u;
#pragma unroll
    for (int u = 0; u < WP; ++u) {
      const char* base = reinterpret_cast<const char*>(W + (rw0 + 2 * u) * n + i1);
      wt[u] = *reinterpret_cast<const floatx4*>(base + woff);
    }
    if (MODE == MODE_FORCED) {
      const uint32_t moff = (uint32_t)((lane >> 5) * n + (lane & 31) * 4);
#pragma unroll
      for (int u = 0; u < WP; ++u) {
        const unsigned char* base = mask_in + (rw0 + 2 * u) * n + i1;
        mw[u] = *reinterpret_cast<const unsigned*>(base + moff);
      }
    }
  } else if (vio) {
#pragma unroll
    for (int u = 0; u < WP; ++u) {
      const int f = u * 64 + lane, rr = f >> 5, c4 = (f & 31) * 4;
      const int64_t r = rw0 + rr < m ? rw0 + rr : m - 1;
      wt[u] = *reinterpret_cast<const floatx4*>(W + r * n + i1 + (c4 < w ? c4 : w - 4));
    }
    if (MODE == MODE_FORCED) {
#pragma unroll
      for (int u = 0; u < WP; ++u) {
        const int f = u * 64 + lane, rr = f >> 5, c4 = (f & 31) * 4;
        const int64_t r = rw0 + rr < m ? rw0 + rr : m - 1;
        mw[u] = *reinterpret_cast<const unsigned*>(mask_in + r * n + i1 + (c4 < w ? c4 : w - 4));
      }
    }
  }

  // threshold key of the block (the LDS of the U block serves as scratch)
  __shared__ unsigned s_cnt;
  __shared__ HistPick s_pick;
  unsigned long long thr = 0ull;
  if (MODE == MODE_THRESH && sel_fixed == 0)
    thr = select_finish(stp->set[parity], candp, ksel, reinterpret_cast<unsigned long long*>(S.Ub),
                        &s_cnt, s_pick);
  if (MODE == MODE_THRESH && (int)blockIdx.x == segs.wg0[seg]) sel_clear_set(stp->set[parity ^ 1], tid, 256);

  // U block to LDS: entries outside the upper triangle of the w x w block
  // are stored as zero
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int f = u * 256 + tid;
    const int j = f >> 5, c4 = (f & 31) * 4;
    floatx4 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c4 + e;
      t[e] = (j < w && c < w && c >= j) ? uv[u][e] : 0.f;
    }
    *reinterpret_cast<floatx4*>(&S.Ub[j * SWS + c4]) = t;
  }
  if (tid < SB) S.Rd[tid] = (tid < w) ? 1.f / udiag : 0.f;

  if (vio) {
#pragma unroll
    for (int u = 0; u < WP; ++u) {
      const int f = u * 64 + lane, rr = f >> 5, c4 = (f & 31) * 4;
      *reinterpret_cast<floatx4*>(&Tw[rr * SWS + c4]) = c4 < w ? wt[u] : floatx4{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) Wt[c][v] = v < RPL ? Tw[(RPL * lg + v) * SWS + 16 * c + lc] : 0.f;
    __builtin_amdgcn_wave_barrier();
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col = 16 * c + lc;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t r = rowok[v] ? r0 + v : m - 1;
        Wt[c][v] = (v < RPL && col < w) ? W[r * n + i1 + (col < w ? col : 0)] : 0.f;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    Et[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    Pm[c] = 0u;
  }
  __syncthreads();
  if constexpr (JOINT) {
    // Gram U16^T U16 of each chunk's diagonal block (U is upper triangular)
    for (int f = tid; f < 8 * 256; f += 256) {
      const int cc = f >> 8, i = (f >> 4) & 15, j = f & 15;
      const int lo = i < j ? i : j;
      float acc = 0.f;
      for (int b = 0; b <= lo; ++b)
        acc = fmaf(S.Ub[(16 * cc + b) * SWS + 16 * cc + i], S.Ub[(16 * cc + b) * SWS + 16 * cc + j], acc);
      S.Gc[cc][i * GCS + j] = acc;
    }
    __syncthreads();
  }

  // masks known at the block start
  if (MODE == MODE_FORCED) {
    if (vio) {
      // the wave's RW x w mask bytes (loaded in the prologue, 4 bytes per
      // access) through the staging tile
      unsigned* Tb = reinterpret_cast<unsigned*>(Tw);
#pragma unroll
      for (int u = 0; u < WP; ++u) {
        const int f = u * 64 + lane, rr = f >> 5, c4 = (f & 31) * 4;
        Tb[rr * 32 + (c4 >> 2)] = c4 < w ? mw[u] : 0u;
      }
      __builtin_amdgcn_wave_barrier();
      const unsigned char* Tm = reinterpret_cast<const unsigned char*>(Tw);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < RPL; ++v)
          if (rowok[v] && Tm[(RPL * lg + v) * 128 + 16 * c + lc] != 0) Pm[c] |= 1u << v;
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int col = 16 * c + lc;
#pragma unroll
        for (int v = 0; v < RPL; ++v)
          if (rowok[v] && col < w && mask_in[(r0 + v) * n + i1 + col] != 0) Pm[c] |= 1u << v;
      }
    }
  } else if (MODE == MODE_THRESH) {
    // key <= thr as one 64-bit compare per key (saliency bits, then the
    // position r*n + c modulo 2^32 as in sal_key); the uniform cases (none
    // or all selected) branch once, outside the loops.  The eight 1/U_cc
    // values are read before any is used.
    const unsigned rows = (rowok[0] ? 1u : 0u) | (rowok[1] ? 2u : 0u) | (rowok[2] ? 4u : 0u) |
                          (rowok[3] ? 8u : 0u);
    if (sel_fixed == 0) {
      const uint32_t lin0 = (uint32_t)(r0 * n + i1 + lc), nn = (uint32_t)n;
      float rdv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) rdv[c] = S.Rd[16 * c + lc];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        unsigned bits = 0u;
#pragma unroll
        for (int v = 0; v < RPL; ++v) {
          const uint32_t lin = lin0 + (uint32_t)v * nn + 16u * (uint32_t)c;
          const unsigned long long key =
              ((unsigned long long)__float_as_uint(saliency(Wt[c][v], rdv[c])) << 32) | lin;
          bits |= (key <= thr ? 1u : 0u) << v;
        }
        Pm[c] |= bits & (16 * c + lc < w ? rows : 0u);
      }
    } else if (sel_fixed == 3) {
#pragma unroll
      for (int c = 0; c < 8; ++c) Pm[c] |= 16 * c + lc < w ? rows : 0u;
    }
  }

  float* Es = S.Es[wave];
  // groups of M <= 16 are ranked inside the column steps (MGS = M); larger
  // groups (and the per-row mode, whose group is the whole block: mgroup = w)
  // at their first chunk, from the saliencies of all their chunks
  const bool nm_large = (MODE == MODE_NM && MGS == 0) || MODE == MODE_ROW;
  const unsigned rowbits = (rowok[0] ? 1u : 0u) | (rowok[1] ? 2u : 0u) | (rowok[2] ? 4u : 0u) |
                           (rowok[3] ? 8u : 0u);
  // Constants of chunk c (every lane reads all 16 values: no per-lane branch
  // around a read).  Chunks past the block read zeros of the U block.
  auto chunk_ctx = [&](int c) {
    ChunkCtx cx;
    const int col = 16 * c + lc;
    cx.ucc = S.Ub[col * SWS + col];
    cx.rd = S.Rd[col];  // 1 / U_col,col, 0 past the block
    float rdj[16], uj[16];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const floatx4 t = *reinterpret_cast<const floatx4*>(&S.Rd[16 * c + 4 * j4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) rdj[4 * j4 + e] = t[e];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) uj[j] = S.Ub[(16 * c + j) * SWS + col];
#pragma unroll
    for (int j = 0; j < 16; ++j) cx.g[j] = (j == lc) ? 0.f : uj[j] * rdj[j];
    return cx;
  };
  // Software pipeline over the chunks: the errors of chunk c update chunk
  // c + 1 at once (its steps wait on that), and the chunks after it during
  // chunk c + 1's steps, which touch none of them, so the matrix core works
  // beside the serial column chain.  Modes that rank whole groups of later
  // chunks at a chunk start need every update first and keep the plain order.
  constexpr bool kDefer = !((MODE == MODE_NM && MGS == 0) || MODE == MODE_ROW);
  floatx4 ead = floatx4{0.f, 0.f, 0.f, 0.f};
  float bvd[8][4];
  ChunkCtx cx = chunk_ctx(0);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c >= nch) break;
    // the next chunk's constants now: their LDS latency hides behind the steps
    ChunkCtx cxn;
    if (c + 1 < 8) cxn = chunk_ctx(c + 1);
    if constexpr (kDefer) {
      // E_{c-1} U[c-1, c'] for the chunks c' after this one
      if (c >= 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c2 = 2; c2 < 8; ++c2) {
            if (c2 <= c) continue;
            Wt[c2] = __builtin_amdgcn_mfma_f32_16x16x4f32(-ead[i], bvd[c2][i], Wt[c2], 0, 0, 0);
          }
      }
    }
    if (nm_large && ((16 * c) % mgroup) == 0) {
      // group of mgroup columns = chunks c .. c + ceil(mgroup/16) - 1 (all current)
      const int nchg = (mgroup + 15) >> 4;
      const int kp = mgroup - nkeep;  // pruned per row
      if (mgroup > 64) {
        // k-th smallest 39-bit key (saliency bits, position) per row by a
        // bitwise search: counts over the 16 lanes of the row by DPP sums
        unsigned long long key[8][4];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const int pos = 16 * g + lc;
          const int col = 16 * (c + g) + lc;
          const bool ok = g < nchg && c + g < 8 && pos < mgroup;
          const float rdg = S.Rd[ok ? col : 0];
#pragma unroll
          for (int v = 0; v < RPL; ++v)
            key[g][v] = ok ? (((unsigned long long)__float_as_uint(saliency(Wt[c + g < 8 ? c + g : 7][v], rdg))
                               << 7) | (unsigned)pos)
                           : ~0ull;
        }
        unsigned long long T[4] = {0ull, 0ull, 0ull, 0ull};
        for (int b = 38; b >= 0; --b) {
#pragma unroll
          for (int v = 0; v < RPL; ++v) {
            const unsigned long long cand = T[v] | (1ull << b);
            int cnt = 0;
#pragma unroll
            for (int g = 0; g < 8; ++g) cnt += key[g][v] < cand ? 1 : 0;
            if (rowsum16(cnt) < kp) T[v] = cand;
          }
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          if (c + g >= 8) continue;
#pragma unroll
          for (int v = 0; v < RPL; ++v)
            if (rowok[v] && kp > 0 && key[g][v] <= T[v]) Pm[c + g] |= 1u << v;
        }
      } else {
        float* sc = Tw;
        for (int g = 0; g < nchg && c + g < 8; ++g) {
          const int col = 16 * (c + g) + lc;
          const float rdg = S.Rd[col];
#pragma unroll
          for (int v = 0; v < RPL; ++v) sc[(RPL * lg + v) * SWS + 16 * g + lc] = saliency(Wt[c + g][v], rdg);
        }
        __builtin_amdgcn_wave_barrier();
        for (int g = 0; g < nchg && c + g < 8; ++g) {
#pragma unroll
          for (int v = 0; v < RPL; ++v) {
            const float* row = sc + (RPL * lg + v) * SWS;
            const int me = 16 * g + lc;
            if (rowok[v] && me < mgroup && rank_of(row, mgroup, row[me], me) < kp)
              Pm[c + g] |= 1u << v;
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    float ev[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (JOINT)
      joint_chunk<MGS, RPL>(std::make_integer_sequence<int, 16>{}, Wt[c], Pm[c], cx, lc, lg, nkeep, rowbits,
                       S.Gc[c], &S.Ub[(16 * c + lc) * SWS + 16 * c], ev);
    else
      sweep_chunk<MGS, QUANT, RPL>(std::make_integer_sequence<int, 16>{}, Wt[c], Pm[c], cx, lc, nkeep, rowbits,
                                   q);
    // errors of the chunk: e = (W_J - target) / U_JJ, from the frozen owner
    // values; pruned entries become +0.0, quantized ones their grid value
#pragma unroll
    for (int v = 0; v < RPL; ++v) {
      const bool p = (Pm[c] >> v) & 1u;
      if constexpr (JOINT) {
        Et[c][v] = ev[v];
        Wt[c][v] = p ? 0.f : fmaf(-ev[v], cx.ucc, Wt[c][v]);
      } else if constexpr (QUANT) {
        const float t = quant_value(Wt[c][v], q, v);
        Et[c][v] = (p ? Wt[c][v] : Wt[c][v] - t) * cx.rd;
        Wt[c][v] = p ? 0.f : t;
      } else {
        Et[c][v] = p ? Wt[c][v] * cx.rd : 0.f;
        Wt[c][v] = p ? 0.f : Wt[c][v];
      }
    }
    if constexpr (kDefer) {
      // issue order: each deferred MFMA between a few of the steps' VALU
      // instructions, from the chunk start on
      if (c >= 1) {
#pragma unroll
        for (int k = 0; k < 4 * (7 - c); ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
      }
    }
    if (c + 1 < 8 && c + 1 < nch) {
      // E_c to the A-operand layout: Es[row][4*(k%4) + k/4] so that lane l
      // reads E[l%16][4*i + l/16] for i = 0..3 as one 16-byte value
#pragma unroll
      for (int v = 0; v < 4; ++v) Es[(4 * lg + v) * ESS + 4 * (lc & 3) + (lc >> 2)] = Et[c][v];
      // one wave writes and reads its own tile: its LDS operations execute in
      // order, so no wait is needed between them (as for the W staging)
      __builtin_amdgcn_wave_barrier();
      const floatx4 ea = *reinterpret_cast<const floatx4*>(&Es[lc * ESS + 4 * lg]);
      __builtin_amdgcn_wave_barrier();
      // B operands first (one wait), then the MFMAs
      float bv[8][4];
#pragma unroll
      for (int c2 = 1; c2 < 8; ++c2) {
        if (c2 <= c) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[c2][i] = S.Ub[(16 * c + 4 * i + lg) * SWS + 16 * c2 + lc];
      }
      if constexpr (kDefer) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Wt[c + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(-ea[i], bv[c + 1][i], Wt[c + 1], 0, 0, 0);
        ead = ea;
#pragma unroll
        for (int c2 = 2; c2 < 8; ++c2) {
          if (c2 <= c + 1) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) bvd[c2][i] = bv[c2][i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c2 = 1; c2 < 8; ++c2) {
            if (c2 <= c) continue;
            Wt[c2] = __builtin_amdgcn_mfma_f32_16x16x4f32(-ea[i], bv[c2][i], Wt[c2], 0, 0, 0);
          }
      }
    }
    if (c + 1 < 8) cx = cxn;
  }

  // retire the block: W (pruned entries +0.0), errors, mask, straight from
  // the registers (each store instruction writes 16 consecutive values of
  // four row groups; no staging round trip through LDS).  Full blocks of full
  // rows store from RPL row pointers with constant offsets.
  if (w == SB && rw0 + RW <= m) {
    float* wr[RPL];
    float* er[RPL];
    uint8_t* mr[RPL];
    uint8_t* qr[RPL];
#pragma unroll
    for (int v = 0; v < RPL; ++v) {
      const int64_t r = r0 + v;
      wr[v] = W + r * n + i1 + lc;
      er[v] = Err + r * EGK + lc;
      mr[v] = mask_out ? mask_out + r * n + i1 + lc : nullptr;
      qr[v] = (QUANT && codes_out) ? codes_out + r * n + i1 + lc : nullptr;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int v = 0; v < RPL; ++v) {
        wr[v][16 * c] = Wt[c][v];
        er[v][16 * c] = Et[c][v];
      }
    if (mask_out) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < RPL; ++v) mr[v][16 * c] = (uint8_t)((Pm[c] >> v) & 1u);
    }
    if (QUANT && codes_out) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < RPL; ++v)
          qr[v][16 * c] = (unsigned char)fminf(fmaxf(rintf(Wt[c][v] * q.inv[v]) + q.z[v], 0.f), q.L);
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int col = 16 * c + lc;
    if (col >= w) continue;
#pragma unroll
    for (int v = 0; v < RPL; ++v) {
      if (!rowok[v]) continue;
      const int64_t r = r0 + v;
      const bool p = (Pm[c] >> v) & 1u;
      W[r * n + i1 + col] = Wt[c][v];
      if (mask_out) mask_out[r * n + i1 + col] = p ? 1 : 0;
      if (QUANT && codes_out)
        codes_out[r * n + i1 + col] =
            (unsigned char)fminf(fmaxf(rintf(Wt[c][v] * q.inv[v]) + q.z[v], 0.f), q.L);
      Err[r * EGK + col] = Et[c][v];
    }
  }
}

// One in-block sweep launch (host side).
struct SweepArgs {
  float* W;
  uint8_t* mask_out;
  float* Err;
  const uint8_t* mask_in;
  SelState* st;
  const unsigned long long* cand;
  int parity;
  Segs segs;
  int64_t n, i1;
  int w, nkeep, mgroup;
  uint8_t* codes_out;
  const float* qscale;
  const float* qzero;
  float qlevels;
  int mode;   // MODE_*
  int mgs;    // N:M groups ranked inside the column steps (1, 2, 4, 8, 16), else 0
  int rpl;    // rows per lane, 4 or 2 (segs.wg0 counts 16 * rpl rows a workgroup)
  dim3 grid;
  hipStream_t stream;
};

sg_status launch_sweep_plain(const SweepArgs& a);  // column by column, no grid
sg_status launch_sweep_quant(const SweepArgs& a);  // kept weights rounded to the row grid
sg_status launch_sweep_joint(const SweepArgs& a);  // vector-level, 16-column ranges

}  // namespace sg
