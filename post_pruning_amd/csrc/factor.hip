// U = upper Cholesky factor of (H + lambda I)^{-1}, lambda = damp * mean(diag H).
//
// The review of "SparseGPT ... Pruned in One-Shot" (devpress), section 8,
// derives each removal's error and the compensation of the remaining weights
// from the inverse Hessian; the pages do not say how that inverse is formed.
// Reading adopted: H_d = H + lambda I, and U with U^T U = H_d^{-1}, U upper
// triangular with a positive diagonal (row j of U then carries the inverse
// Hessian of the columns j..n-1 still free when column j is processed).
//
// Route on the GPU (fp32 throughout):
//   A = J H_d J            (J reverses indices; fused into the damping copy)
//   A = L L^T              (blocked right-looking Cholesky, panel width 128)
//   Y = L^{-T}             (the triangular inverse, carried along the same
//                           panel loop: block column k of Y is finished by the
//                           same panel that finishes block column k of L)
//   U = J L^{-1} J, i.e. U[i][j] = Y[n-1-j][n-1-i]
// Since J H_d J = L L^T gives H_d = (J L J)(J L J)^T with J L J upper, its
// inverse is (J L^{-1} J)^T (J L^{-1} J): U = J L^{-1} J is exactly the upper
// factor of H_d^{-1}.  Algorithmic work n^3/3 (Cholesky) + n^3/3 (inverse).
//
// Per panel k (block size NB = 128, matrix padded to n_pad = 128 * nblk with
// an identity tail):
//   panel kernel: every workgroup factors A_kk in LDS and inverts it, then
//     row blocks l > k:  L[l,k] = A[l,k] * L_kk^{-T}                 (TRSM)
//     col blocks c < k:  Y[c,k] = R[c,k] * L_kk^{-T}                 (inverse)
//     c == k:            Y[k,k] = L_kk^{-T}
//   trailing update (fp32-accurate products on bf16 MFMA, K = 128):
//     A[l,m] -= L[l,k] L[m,k]^T   for k < m <= l                     (SYRK)
//     R[c,l] -= Y[c,k] L[l,k]^T   for c <= k < l                      (inverse)
// where R is the running right-hand side of L X = I, kept transposed in the
// upper block triangle of Y (R starts as I).  Look-ahead: block column k+1
// of the update goes first (one short launch); panel k+1 then runs on the
// caller's stream while the rest of the update runs beside it (in the same
// launch up to n = 4096, else on a second stream the caller provides).
#include "gemm_x6.h"

#include <math.h>

#include <algorithm>

namespace sg {
namespace {

constexpr int NB = kFactorNB;  // 128

// The matrices of one call, all of order n.  Layer L works in its own part of
// the workspace (ls floats apart): A and Y of n_pad x n_pad, then lambda.
// Every kernel below handles all layers of a call in one launch: its grid is
// the single-layer grid repeated once per layer (or, for the damping and the
// flip copies, one more grid dimension).
struct FactorLayers {
  int nl;
  int64_t ls;
  const float* H[SG_MAX_SEGMENTS];
  float* Hinv[SG_MAX_SEGMENTS];
  int32_t* info[SG_MAX_SEGMENTS];
};

// ---- damping --------------------------------------------------------------
// One workgroup of 1024 threads; each thread's diagonal entries (one cache
// line apiece) are requested eight at a time before they are summed.
__global__ __launch_bounds__(1024) void damp_lambda_kernel(const FactorLayers fl, float* ws, int64_t n,
                                                           int64_t n_pad, double damp) {
  const int L = blockIdx.x;
  const float* __restrict__ H = fl.H[L];
  float* lam_out = ws + L * fl.ls + 2 * n_pad * n_pad;
  int32_t* info = fl.info[L];
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += 8 * 1024) {
    float d[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + u * 1024;
      d[u] = i < n ? H[i * n + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s += (double)d[u];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = red[0] / (double)n;
    const double lam = damp * mean;
    const bool ok = isfinite(mean) && mean > 0.0 && isfinite(lam) && lam >= 0.0;
    *info = ok ? 0 : (int32_t)(n + 1);
    *lam_out = ok ? (float)lam : 0.f;
  }
}

// A = J (H + lam I) J on the lower block triangle (identity tail for padding);
// Y = I (zero below the diagonal, so its lower block triangle is zero too:
// the grouped updates read Y[c][k .. c-1]).  64x64 tiles.
__global__ __launch_bounds__(256) void flip_init_kernel(const FactorLayers fl, float* ws, int64_t n,
                                                        int64_t n_pad) {
  const int L = blockIdx.z;
  const float* __restrict__ H = fl.H[L];
  float* __restrict__ A = ws + L * fl.ls;
  float* __restrict__ Y = A + n_pad * n_pad;
  const float* __restrict__ lam_p = Y + n_pad * n_pad;
  const int64_t ti = blockIdx.y, tj = blockIdx.x;
  const float lam = *lam_p;
  const int c = threadIdx.x & 63;
  const int r0 = threadIdx.x >> 6;
  const int64_t j = tj * 64 + c;
  // block-triangle membership at the 128 granularity of the factorisation
  const bool lower = (ti / 2) >= (tj / 2);
  for (int rr = r0; rr < 64; rr += 4) {
    const int64_t i = ti * 64 + rr;
    if (lower) {
      float v;
      if (i < n && j < n) {
        v = H[(n - 1 - i) * n + (n - 1 - j)];
        if (i == j) v += lam;
      } else {
        v = (i == j) ? 1.f : 0.f;
      }
      A[i * n_pad + j] = v;
    }
    Y[i * n_pad + j] = (i == j) ? 1.f : 0.f;
  }
}

// ---- panel ---------------------------------------------------------------
// The diagonal block A_kk (128 x 128) is factored and inverted inside one
// workgroup with a blocked algorithm of 16-column sub-panels:
//   * wave 0 factors sub-panel p (rows 16p..127, 16 columns) in registers, the
//     pivot row's entries broadcast with readlane (no LDS round trip);
//   * all waves apply its rank-16 update to the trailing lower triangle with
//     v_mfma_f32_16x16x4_f32 directly out of LDS;
//   * the 16x16 diagonal blocks of L_kk^{-1} are formed by forward
//     substitution (one lane per column), the off-diagonal blocks by block
//     forward substitution X[P][Q] = -D_P sum_{R=Q}^{P-1} L[P][R] X[R][Q] on
//     MFMA (the D-layout of the sum is directly the B operand of the product
//     with D_P).
constexpr int PS = 132;  // LDS row stride (floats): 16-byte rows, conflict-free b128 reads

struct PanelLds {
  float As[NB * PS];  // A_kk / L_kk, later the block to transform
  float Li[NB * PS];
  int fail;
};

// Empty asm that takes the 16 values as read-write operands: they must be
// computed at this point (no instructions are emitted).
__device__ __forceinline__ void pin16(float (&a)[16]) {
  asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
               "+v"(a[6]), "+v"(a[7]));
  asm volatile("" : "+v"(a[8]), "+v"(a[9]), "+v"(a[10]), "+v"(a[11]), "+v"(a[12]), "+v"(a[13]),
               "+v"(a[14]), "+v"(a[15]));
}

__device__ __forceinline__ float rdlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Part of the rank-16 update of the trailing lower triangle after sub-panel
// p: the 16x16 tiles (I, C) of block column q0 (COL: q0 <= I < 8) or of the
// triangle q0 <= C <= I < 8, dealt round robin to NW waves (w = this wave's
// place among them), MT = the most any wave gets.  A wave issues all its LDS
// reads, then its MFMA chains interleaved, then its writes (one LDS round
// trip instead of one per tile); slots past the tile count recompute the
// first tile and are not written.
// Sub-panel factorisation in one wave: the 16 columns c0 .. c0+15 of the
// rows c0 .. 127 (row c0 + lane in a0 and, with TWO, row c0 + 64 + lane in
// a1), pivot by pivot, the pivot row's entries broadcast with readlane.
template <bool TWO>
__device__ __forceinline__ void subpanel_factor(PanelLds& S, int c0, int lane) {
  const int r0 = c0 + lane, r1 = c0 + 64 + lane;
  // 16-byte reads from clamped rows, out-of-range rows zeroed afterwards
  const int r0c = r0 < NB ? r0 : NB - 1, r1c = r1 < NB ? r1 : NB - 1;
  floatx4 t0[4], t1[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t0[q] = *reinterpret_cast<const floatx4*>(&S.As[r0c * PS + c0 + 4 * q]);
    if (TWO) t1[q] = *reinterpret_cast<const floatx4*>(&S.As[r1c * PS + c0 + 4 * q]);
  }
  float a0[16], a1[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    a0[c] = (r0 < NB) ? t0[c >> 2][c & 3] : 0.f;
    a1[c] = (TWO && r1 < NB) ? t1[c >> 2][c & 3] : 0.f;
  }
  // No lane masks: entries above the diagonal start as zero, so scaling
  // column j on every lane leaves them zero and turns the pivot into
  // d2/d = d; the updates below only dirty entries (row j, column > j)
  // above the diagonal, which are never read again and are dropped when
  // the sub-panel is written back.
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float d2 = rdlane(a0[j], j);
    // hardware reciprocal square root (about 1 ulp): the pivot chain is the
    // latency-critical path of the whole factorisation
    const float rd = __builtin_amdgcn_rsqf(d2);
    a0[j] *= rd;
    if (TWO) a1[j] *= rd;
#pragma unroll
    for (int c = j + 1; c < 16; ++c) {
      const float lcj = rdlane(a0[j], c);
      a0[c] = fmaf(-a0[j], lcj, a0[c]);
      if (TWO) a1[c] = fmaf(-a1[j], lcj, a1[c]);
    }
    // right-looking order: the updated columns are materialised after
    // every step, so each broadcast is consumed in its own step (left to
    // itself the compiler sinks the updates to their first use and keeps
    // every broadcast value live in scalar registers, which spill)
    pin16(a0);
    if (TWO) pin16(a1);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    floatx4 w0, w1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0[e] = (4 * q + e <= lane) ? a0[4 * q + e] : 0.f;
      w1[e] = a1[4 * q + e];
    }
    if (r0 < NB) *reinterpret_cast<floatx4*>(&S.As[r0 * PS + c0 + 4 * q]) = w0;
    if (TWO && r1 < NB) *reinterpret_cast<floatx4*>(&S.As[r1 * PS + c0 + 4 * q]) = w1;
  }
  // breakdown: a pivot that was not positive and finite leaves a diagonal
  // entry that is not (0 * inf, NaN or inf), and every later one follows;
  // the first such column of the sub-panel is recorded
  const float dj = S.As[(c0 + (lane & 15)) * PS + c0 + (lane & 15)];
  const unsigned long long bad = __ballot(lane < 16 && !(dj > 0.f && isfinite(dj)));
  if (lane == 0 && bad != 0ull && S.fail < 0) S.fail = c0 + __builtin_ctzll(bad);
}

// Row index ii of triangle tile idx (idx = ii (ii + 1) / 2 + cc, 0 <= cc <= ii),
// 3 bits per entry: tiles 0..20 in kTriLo, 21..27 in kTriHi.
constexpr uint64_t kTriLo = 0x5b6db2491b6d2448ull;
constexpr uint64_t kTriHi = 0x1b6db6ull;

template <int MT, bool COL, int NW>
__device__ __forceinline__ void rank16_update(PanelLds& S, int p, int q0, int w, int lane) {
  const int c0 = 16 * p;
  const int t = 8 - q0;
  const int ntiles = COL ? t : t * (t + 1) / 2;
  floatx4 acc[MT], fa[MT], fb[MT];
  int aoff[MT];
#pragma unroll
  for (int s = 0; s < MT; ++s) {
    const int i0 = w + NW * s;
    const int idx = i0 < ntiles ? i0 : 0;
    // tile idx = ii (ii + 1) / 2 + cc of the triangle: ii from a packed
    // table of 3-bit entries (idx < 28), no search loop
    const int ii = COL ? idx : (int)((idx < 21 ? (kTriLo >> (3 * idx)) : (kTriHi >> (3 * (idx - 21)))) & 7u);
    const int cc = COL ? 0 : idx - ii * (ii + 1) / 2;
    const int I = q0 + ii, C = q0 + cc;
    aoff[s] = (I * 16 + (lane >> 4) * 4) * PS + C * 16 + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[s][v] = S.As[aoff[s] + v * PS];
    fa[s] = *reinterpret_cast<const floatx4*>(&S.As[(I * 16 + (lane & 15)) * PS + c0 + (lane >> 4) * 4]);
    fb[s] = *reinterpret_cast<const floatx4*>(&S.As[(C * 16 + (lane & 15)) * PS + c0 + (lane >> 4) * 4]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int s = 0; s < MT; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(-fa[s][e], fb[s][e], acc[s], 0, 0, 0);
#pragma unroll
  for (int s = 0; s < MT; ++s)
    if (w + NW * s < ntiles) {
#pragma unroll
      for (int v = 0; v < 4; ++v) S.As[aoff[s] + v * PS] = acc[s][v];
    }
}

// Column blocks Q1 and Q2 of X = L_kk^{-1} below the diagonal, formed by one
// wave: X[P][Q] = -D_P sum_{R=Q}^{P-1} L[P][R] X[R][Q] for P = Q+1 .. 7 in
// order, D_P = X[P][P] (the 16x16 diagonal inverses, already in Li).  A
// column's blocks depend only on blocks of the same column, so the wave needs
// no barrier between them: each block stays in registers, where its MFMA
// result layout (lane l, value v: row 4(l/16)+v, column l%16) is exactly the
// B operand the later products read (k = 4(l/16)+e for the e-th K=4 MFMA),
// and is written to Li for the apply.  The two columns' chains interleave.
template <int Q1, int Q2>
__device__ __forceinline__ void inv_columns(PanelLds& S, int lane) {
  floatx4 X1[8], X2[8];
  const int lr = lane & 15, lk = (lane >> 4) * 4;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    X1[Q1][v] = S.Li[(Q1 * 16 + lk + v) * PS + Q1 * 16 + lr];
    X2[Q2][v] = S.Li[(Q2 * 16 + lk + v) * PS + Q2 * 16 + lr];
  }
#pragma unroll
  for (int P = 1; P < 8; ++P) {
    if (P <= Q1 && P <= Q2) continue;
    // the row P fragments of L (A operands, 4 consecutive k per lane)
    floatx4 fa[8];
#pragma unroll
    for (int R = 0; R < P; ++R)
      if (R >= (Q1 < Q2 ? Q1 : Q2))
        fa[R] = *reinterpret_cast<const floatx4*>(&S.As[(P * 16 + lr) * PS + R * 16 + lk]);
    const floatx4 fd = *reinterpret_cast<const floatx4*>(&S.Li[(P * 16 + lr) * PS + P * 16 + lk]);
    floatx4 T1 = floatx4{0.f, 0.f, 0.f, 0.f}, T2 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int R = 0; R < P; ++R)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (P > Q1 && R >= Q1) T1 = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[R][e], X1[R][e], T1, 0, 0, 0);
        if (P > Q2 && R >= Q2) T2 = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[R][e], X2[R][e], T2, 0, 0, 0);
      }
    floatx4 Y1 = floatx4{0.f, 0.f, 0.f, 0.f}, Y2 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (P > Q1) Y1 = __builtin_amdgcn_mfma_f32_16x16x4f32(-fd[e], T1[e], Y1, 0, 0, 0);
      if (P > Q2) Y2 = __builtin_amdgcn_mfma_f32_16x16x4f32(-fd[e], T2[e], Y2, 0, 0, 0);
    }
    if (P > Q1) {
      X1[P] = Y1;
#pragma unroll
      for (int v = 0; v < 4; ++v) S.Li[(P * 16 + lk + v) * PS + Q1 * 16 + lr] = Y1[v];
    }
    if (P > Q2) {
      X2[P] = Y2;
#pragma unroll
      for (int v = 0; v < 4; ++v) S.Li[(P * 16 + lk + v) * PS + Q2 * 16 + lr] = Y2[v];
    }
  }
}

// R = rows of the block this workgroup transforms at the end (128 / R
// workgroups share each block; every one of them factors A_kk).
template <int R>
__device__ __forceinline__ void panel_body(PanelLds& S, float* __restrict__ A, float* __restrict__ Y,
                                           int64_t n_pad, int k, int64_t n, int32_t* info, int b, int part) {
  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: held in a scalar register
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t k0 = (int64_t)k * NB;

  // The R x 128 part of the block this workgroup transforms at the end
  // (rows part * R ..) is fetched into registers right away, so its latency
  // hides behind the factorisation.
  float* blk = nullptr;
  if (b > k)
    blk = A + ((int64_t)b * NB + part * R) * n_pad + k0;  // L[l,k] = A[l,k] L_kk^{-T}
  else if (b < k)
    blk = Y + ((int64_t)b * NB + part * R) * n_pad + k0;  // Y[c,k] = R[c,k] L_kk^{-T}
  constexpr int TPR = 256 / R;       // threads per row of the part
  constexpr int CPT = NB / TPR;      // columns per thread
  const int prow_t = tid / TPR, pcol_t = (tid % TPR) * CPT;
  floatx4 bv[CPT / 4];
  if (blk) {
#pragma unroll
    for (int u = 0; u < CPT / 4; ++u)
      bv[u] = *reinterpret_cast<const floatx4*>(blk + (int64_t)prow_t * n_pad + pcol_t + 4 * u);
  }
  const int brow = tid >> 1, bcol = (tid & 1) * 64;

  // 0. load the lower part of A_kk (all loads issued together), clear L_kk^{-1}
  {
    floatx4 av[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      av[u] = *reinterpret_cast<const floatx4*>(A + (k0 + brow) * n_pad + k0 + bcol + 4 * u);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      floatx4 v = av[u];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (bcol + 4 * u + e > brow) v[e] = 0.f;
      *reinterpret_cast<floatx4*>(&S.As[brow * PS + bcol + 4 * u]) = v;
      *reinterpret_cast<floatx4*>(&S.Li[brow * PS + bcol + 4 * u]) = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (tid == 0) S.fail = -1;
  __syncthreads();

  // 1. blocked Cholesky, 16-column sub-panels, with a look-ahead of one:
  // after sub-panel p, the four waves first update block column p+1 (what
  // sub-panel p+1 reads); then wave 0 factors sub-panel p+1 while waves 1..3
  // update the rest of the trailing triangle (block columns p+2 ..), which
  // sub-panel p+1 neither reads nor writes.
  if (wave == 0) subpanel_factor<true>(S, 0, lane);
  __syncthreads();
  for (int p = 0; p < 7; ++p) {
    // block column p+1: 7 - p tiles
    if (p < 3)
      rank16_update<2, true, 4>(S, p, p + 1, wave, lane);
    else
      rank16_update<1, true, 4>(S, p, p + 1, wave, lane);
    __syncthreads();
    if (wave == 0) {
      // rows c0 + lane and, while they exist, c0 + 64 + lane
      const int c0 = (p + 1) * 16;
      if (c0 + 64 < NB)
        subpanel_factor<true>(S, c0, lane);
      else
        subpanel_factor<false>(S, c0, lane);
    } else {
      // the triangle of block columns p+2 .. 7: (6 - p)(7 - p)/2 tiles
      switch (p) {
        case 0: rank16_update<7, false, 3>(S, p, p + 2, wave - 1, lane); break;
        case 1: rank16_update<5, false, 3>(S, p, p + 2, wave - 1, lane); break;
        case 2: rank16_update<4, false, 3>(S, p, p + 2, wave - 1, lane); break;
        case 3: rank16_update<2, false, 3>(S, p, p + 2, wave - 1, lane); break;
        case 4:
        case 5: rank16_update<1, false, 3>(S, p, p + 2, wave - 1, lane); break;
        default: break;
      }
    }
    __syncthreads();
  }
  if (b == 0 && part == 0 && tid == 0 && S.fail >= 0) {
    const int64_t pcol = k0 + S.fail;  // column in the flipped order
    if (pcol < n) atomicCAS(info, 0, (int32_t)(n - pcol));
  }

  // 2a. inverses of the 16x16 diagonal blocks: lane -> (block, column)
  if (lane < 32) {
    const int P = wave * 2 + (lane >> 4);
    const int c = lane & 15;
    const int b0 = P * 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < i; ++q) acc = fmaf(S.As[(b0 + i) * PS + b0 + q], x[q], acc);
      const float rlii = __builtin_amdgcn_rcpf(S.As[(b0 + i) * PS + b0 + i]);
      x[i] = (i < c) ? 0.f : ((i == c) ? rlii : -acc * rlii);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) S.Li[(b0 + i) * PS + b0 + c] = x[i];
  }
  __syncthreads();
  // 2b. the blocks below the diagonal, column block by column block: wave w
  // forms columns w and 7 - w (balanced work, no barrier in between)
  switch (wave) {
    case 0: inv_columns<0, 7>(S, lane); break;
    case 1: inv_columns<1, 6>(S, lane); break;
    case 2: inv_columns<2, 5>(S, lane); break;
    default: inv_columns<3, 4>(S, lane); break;
  }
  __syncthreads();

  // 3. apply
  if (b == k) {
    // Y[k,k] = L_kk^{-T}, rows part * R ..
    for (int e = tid; e < R * NB; e += 256) {
      const int i = part * R + (e >> 7), c = e & 127;
      Y[(k0 + i) * n_pad + k0 + c] = S.Li[c * PS + i];
    }
    return;
  }
  // stage the prefetched part into the (now free) A_kk area
#pragma unroll
  for (int u = 0; u < CPT / 4; ++u)
    *reinterpret_cast<floatx4*>(&S.As[prow_t * PS + pcol_t + 4 * u]) = bv[u];
  __syncthreads();
  // out[r][c] = sum_q part[r][q] Linv[c][q]: wave w owns output columns
  // 32w .. 32w+31 of all R rows, (R/16) x 2 MFMA blocks
  constexpr int NI = R / 16;
  floatx4 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i) acc[i][0] = acc[i][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int qrow = wave * 32 + (lane & 15);
#pragma unroll 2
  for (int kc = 0; kc < NB; kc += 16) {
    const int kl = kc + (lane >> 4) * 4;
    floatx4 pp[NI], qq[2];
#pragma unroll
    for (int i = 0; i < NI; ++i) pp[i] = *reinterpret_cast<const floatx4*>(&S.As[(i * 16 + (lane & 15)) * PS + kl]);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) qq[jj] = *reinterpret_cast<const floatx4*>(&S.Li[(qrow + jj * 16) * PS + kl]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(pp[i][e], qq[jj][e], acc[i][jj], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        blk[(int64_t)(i * 16 + (lane >> 4) * 4 + v) * n_pad + wave * 32 + jj * 16 + (lane & 15)] = acc[i][jj][v];
}

// ---- trailing update ------------------------------------------------------
__device__ inline int64_t isqrt_floor(int64_t x) {
  int64_t r = (int64_t)sqrt((double)x);
  while (r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r;
}

// Trailing-update tiles of panels k .. kl = k + kw - 1 (K = 128 kw: the
// group's updates in one pass), in three subsets:
//   UPD_ALL   every tile;
//   UPD_COL   the tiles of block column kl+1 only (what panel kl+1 needs;
//             run by col_update_kernel in 64x64 quarters);
//   UPD_REST  every other tile (run beside panel kl+1).
// SYRK tiles (l, m), kl < m <= l: A[l,m] -= L[l,k:kl+1] L[m,k:kl+1]^T.
// Inverse tiles (c, l), c <= kl < l: R[c,l] -= Y[c,k:kl+1] L[l,k:kl+1]^T
// (for c > k the terms Y[c][k .. c-1] lie in Y's lower block triangle,
// which is zero).  Grouping divides the passes over the trailing matrix,
// whose read-modify-write bounds the update at large n, by kw.
enum { UPD_ALL = 0, UPD_COL = 1, UPD_REST = 2 };

__host__ __device__ inline int64_t update_tiles(int k, int kw, int nblk, int mode) {
  const int kl = k + kw - 1;
  const int64_t t = nblk - kl - 1;  // trailing block count
  if (t <= 0) return 0;
  if (mode == UPD_COL) return t + (kl + 1);
  if (mode == UPD_REST) return (t - 1) * t / 2 + (int64_t)(kl + 1) * (t - 1);
  return t * (t + 1) / 2 + (int64_t)(kl + 1) * t;
}

template <int KW>
__device__ __forceinline__ void update_body(float* lds, float* __restrict__ A, float* __restrict__ Y,
                                            int64_t n_pad, int k, int nblk, int mode, int64_t idx) {
  // UPD_ALL or UPD_REST.  SYRK tiles: lower triangle over trailing blocks
  // [s0, nblk); inverse tiles: rows c <= kl, block columns [s0, nblk)
  const int kl = k + KW - 1;
  const int64_t s0 = mode == UPD_REST ? kl + 2 : kl + 1;
  const int64_t ts = nblk - s0;
  const int64_t nsyrk = ts * (ts + 1) / 2;
  float* C;
  const float *P, *Q;
  if (idx < nsyrk) {
    int64_t l = (isqrt_floor(8 * idx + 1) - 1) / 2;
    while ((l + 1) * (l + 2) / 2 <= idx) ++l;
    while (l * (l + 1) / 2 > idx) --l;
    const int64_t m = idx - l * (l + 1) / 2;
    const int64_t lb = s0 + l, mb = s0 + m;
    C = A + lb * NB * n_pad + mb * NB;
    P = A + lb * NB * n_pad + (int64_t)k * NB;
    Q = A + mb * NB * n_pad + (int64_t)k * NB;
  } else {
    idx -= nsyrk;
    const int64_t c = idx % (kl + 1);
    const int64_t lb = s0 + idx / (kl + 1);
    C = Y + c * NB * n_pad + lb * NB;
    P = Y + c * NB * n_pad + (int64_t)k * NB;
    Q = A + lb * NB * n_pad + (int64_t)k * NB;
  }
  // fp32-accurate products on bf16 MFMA (three-way split, six terms); every
  // tile is full (n_pad < 2^24: the workspace holds 2 n_pad^2 floats)
  RowsX6V<NB, true> pl{P, n_pad, NB, KW * NB};
  RowsX6V<NB, true> ql{Q, n_pad, NB, KW * NB};
  TileAcc acc;
  tile_zero(acc);
  tile_gemm_x6(acc, pl, ql, KW * NB, lds);
  tile_sub_from(C, n_pad, NB, NB, acc, lds);
}

template <int R>
__global__ __launch_bounds__(256) void panel_kernel(const FactorLayers fl, float* ws, int64_t n_pad, int k,
                                                    int nblk, int64_t n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int parts = NB / R;
  const int npl = nblk * parts;  // workgroups per layer
  const int L = (int)blockIdx.x / npl, j = (int)blockIdx.x - L * npl;
  float* A = ws + L * fl.ls;
  panel_body<R>(*reinterpret_cast<PanelLds*>(smem), A, A + n_pad * n_pad, n_pad, k, n, fl.info[L], j / parts,
                j % parts);
}

// Block column kl+1 of the update of panels k .. kl = k + KW - 1 (what panel
// kl+1 reads first) in 64x64 quarters of the 128x128 tiles: four times the
// workgroups of the tile grid, which is only t + kl + 1 tiles, for a short
// latency-bound launch.
template <int KW>
__global__ __launch_bounds__(256) void col_update_kernel(float* ws, int64_t ls, int64_t n_pad, int k, int nblk,
                                                         int64_t ncl) {
  __shared__ __attribute__((aligned(16))) unsigned char ldsb[X6Lds<64>::SHORT];
  float* lds = reinterpret_cast<float*>(ldsb);
  // layer L's part of the grid: ncl workgroups
  const int64_t L = blockIdx.x / ncl, bid = blockIdx.x - L * ncl;
  float* __restrict__ A = ws + L * ls;
  float* __restrict__ Y = A + n_pad * n_pad;
  const int kl = k + KW - 1;
  const int64_t t = nblk - kl - 1;
  int64_t idx = bid >> 2;
  const int qr = (int)(bid >> 1) & 1, qc = (int)bid & 1;
  float* C;
  const float *P, *Q;
  if (idx < t) {
    // SYRK tile (kl+1+idx, kl+1); its quarter above the diagonal is not needed
    if (idx == 0 && qr < qc) return;
    const int64_t lb = kl + 1 + idx, mb = kl + 1;
    C = A + lb * NB * n_pad + mb * NB;
    P = A + lb * NB * n_pad + (int64_t)k * NB;
    Q = A + mb * NB * n_pad + (int64_t)k * NB;
  } else {
    // inverse tile (c, kl+1)
    const int64_t c = idx - t, lb = kl + 1;
    C = Y + c * NB * n_pad + lb * NB;
    P = Y + c * NB * n_pad + (int64_t)k * NB;
    Q = A + lb * NB * n_pad + (int64_t)k * NB;
  }
  // the quarter of C and (K = 128) both operands are requested before the
  // first product; K >= 256 streams its chunks two ahead
  float* Cq = C + (int64_t)qr * 64 * n_pad + qc * 64;
  CTileV<64> ct;
  ct.load(Cq, n_pad, 64);
  RowsX6V<64, true> pl{P + (int64_t)qr * 64 * n_pad, n_pad, 64, KW * NB};
  RowsX6V<64, true> ql{Q + (int64_t)qc * 64 * n_pad, n_pad, 64, KW * NB};
  TileAccT<64> acc;
  tile_zero(acc);
  if constexpr (KW == 1)
    tile_gemm_x6_short<64, NB / GBK>(acc, pl, ql, NB, ldsb);
  else
    tile_gemm_x6(acc, pl, ql, KW * NB, ldsb);
  tile_sub_pre(Cq, n_pad, 64, ct, acc, lds);
}

// Look-ahead step in one launch: workgroups [0, nblk * 128 / R) factor panel
// kl+1 and transform its blocks (R rows each) while the others apply the rest
// of the update of panels k .. kl (the tiles outside block column kl+1, which
// panel kl+1 does not read).  The panel's workgroups come first in the grid,
// so they are dispatched first.
template <int R, int KW>
__global__ __launch_bounds__(256) void panel_rest_kernel(const FactorLayers fl, float* ws, int64_t n_pad, int k,
                                                         int nblk, int64_t n, int64_t nrest) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int parts = NB / R;
  // every layer's panel workgroups first, then every layer's update tiles
  const int64_t npl = (int64_t)nblk * parts, bid = blockIdx.x;
  if (bid < fl.nl * npl) {
    const int L = (int)(bid / npl), j = (int)(bid - L * npl);
    float* A = ws + L * fl.ls;
    panel_body<R>(*reinterpret_cast<PanelLds*>(smem), A, A + n_pad * n_pad, n_pad, k + KW, n, fl.info[L],
                  j / parts, j % parts);
  } else {
    const int64_t r = bid - fl.nl * npl, L = r / nrest;
    float* A = ws + L * fl.ls;
    update_body<KW>(reinterpret_cast<float*>(smem), A, A + n_pad * n_pad, n_pad, k, nblk, UPD_REST,
                    r - L * nrest);
  }
}

// The rest of the update of panels k .. k + KW - 1 on its own (the panel
// launch runs beside it on a second stream): 66 KB of LDS per workgroup, two
// per CU.
template <int KW>
__global__ __launch_bounds__(256, 2) void rest_update_kernel(float* ws, int64_t ls, int64_t n_pad, int k, int nblk,
                                                             int64_t nrest) {
  __shared__ __attribute__((aligned(16))) unsigned char ldsb[X6Lds<NB>::SIZE];
  const int64_t L = blockIdx.x / nrest;
  float* A = ws + L * ls;
  update_body<KW>(reinterpret_cast<float*>(ldsb), A, A + n_pad * n_pad, n_pad, k, nblk, UPD_REST,
                  (int64_t)blockIdx.x - L * nrest);
}

// The panel chain (factor A_kk, invert it, transform the block column) is
// the critical path of the factorisation at moderate n.  The transform is
// split over 128 / R workgroups per block (each repeats the 128 x 128
// factorisation, which is latency bound) while that keeps the panel launch
// within one workgroup per CU.
//
// Above n = 4096 the trailing update sets the time, and its read-modify-write
// of the trailing matrix bounds it: panels go in groups of up to KWMAX, so
// that one pass with K = 128 kw replaces kw passes with K = 128.  A group of
// kw panels from k: for j = 1 .. kw - 1, block column k+j by panels k ..
// k+j-1 (K = 128 j) and then panel k+j on its own; block column k+kw by the
// whole group; then panel k+kw beside the rest of the group's update.
constexpr int KWMAX = 4;

// host launchers of the templates by group width (1 .. KWMAX)
sg_status launch_col_update(int kw, const FactorLayers& fl, float* ws, int64_t n_pad, int k, int nblk,
                            hipStream_t st) {
  const int64_t ncl = 4 * update_tiles(k, kw, nblk, UPD_COL);
  const dim3 grid((unsigned)(fl.nl * ncl)), blk(256);
  const int64_t ls = fl.ls;
  switch (kw) {
    case 1: hipLaunchKernelGGL(col_update_kernel<1>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, ncl); break;
    case 2: hipLaunchKernelGGL(col_update_kernel<2>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, ncl); break;
    case 3: hipLaunchKernelGGL(col_update_kernel<3>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, ncl); break;
    default: hipLaunchKernelGGL(col_update_kernel<4>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, ncl); break;
  }
  return check_launch("factor update (next column)");
}

sg_status launch_rest_update(int kw, const FactorLayers& fl, float* ws, int64_t n_pad, int k, int nblk,
                             int64_t rest, hipStream_t st) {
  const dim3 grid((unsigned)(fl.nl * rest)), blk(256);
  const int64_t ls = fl.ls;
  switch (kw) {
    case 1: hipLaunchKernelGGL(rest_update_kernel<1>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, rest); break;
    case 2: hipLaunchKernelGGL(rest_update_kernel<2>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, rest); break;
    case 3: hipLaunchKernelGGL(rest_update_kernel<3>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, rest); break;
    default: hipLaunchKernelGGL(rest_update_kernel<4>, grid, blk, 0, st, ws, ls, n_pad, k, nblk, rest); break;
  }
  return check_launch("factor update (rest)");
}

template <int R>
sg_status launch_panel_rest(int kw, const FactorLayers& fl, float* ws, int64_t n_pad, int k, int nblk, int64_t n,
                            int64_t rest, hipStream_t st) {
  constexpr int parts = NB / R;
  const dim3 grid((unsigned)(fl.nl * ((int64_t)nblk * parts + rest))), blk(256);
  const size_t lds = sizeof(PanelLds);
  switch (kw) {
    case 1: hipLaunchKernelGGL((panel_rest_kernel<R, 1>), grid, blk, lds, st, fl, ws, n_pad, k, nblk, n, rest); break;
    case 2: hipLaunchKernelGGL((panel_rest_kernel<R, 2>), grid, blk, lds, st, fl, ws, n_pad, k, nblk, n, rest); break;
    case 3: hipLaunchKernelGGL((panel_rest_kernel<R, 3>), grid, blk, lds, st, fl, ws, n_pad, k, nblk, n, rest); break;
    default: hipLaunchKernelGGL((panel_rest_kernel<R, 4>), grid, blk, lds, st, fl, ws, n_pad, k, nblk, n, rest); break;
  }
  return check_launch("factor panel + rest of update");
}

// One stream: panel 0, then per group the next-column updates and panels of
// the group, and one launch holding the next panel and the rest of the
// group's update.  GROUPS = false: single panels (kw = 1).
template <int R, bool GROUPS>
sg_status run_factor_fused(const FactorLayers& fl, float* ws, int64_t n_pad, int nblk, int64_t n,
                           hipStream_t st) {
  constexpr int parts = NB / R;
  // the LDS limit is a per-device attribute: set on every call (cheap), so
  // that a call on another device finds it set too
  for (const void* f : {reinterpret_cast<const void*>(panel_kernel<R>),
                        reinterpret_cast<const void*>(panel_rest_kernel<R, 1>),
                        reinterpret_cast<const void*>(panel_rest_kernel<R, 2>),
                        reinterpret_cast<const void*>(panel_rest_kernel<R, 3>),
                        reinterpret_cast<const void*>(panel_rest_kernel<R, 4>)})
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PanelLds)) !=
        hipSuccess)
      return set_error(SG_ERR_HIP, "hipFuncSetAttribute(panel kernels) failed");
  const dim3 pgrid((unsigned)(fl.nl * nblk * parts)), blk(256);
  hipLaunchKernelGGL(panel_kernel<R>, pgrid, blk, sizeof(PanelLds), st, fl, ws, n_pad, 0, nblk, n);
  if (sg_status e = check_launch("factor panel")) return e;
  for (int k = 0; k + 1 < nblk;) {
    const int kw = GROUPS ? std::min(KWMAX, nblk - 1 - k) : 1;
    for (int j = 1; j < kw; ++j) {
      if (sg_status e = launch_col_update(j, fl, ws, n_pad, k, nblk, st)) return e;
      hipLaunchKernelGGL(panel_kernel<R>, pgrid, blk, sizeof(PanelLds), st, fl, ws, n_pad, k + j, nblk, n);
      if (sg_status e = check_launch("factor panel")) return e;
    }
    if (sg_status e = launch_col_update(kw, fl, ws, n_pad, k, nblk, st)) return e;
    if (sg_status e = launch_panel_rest<R>(kw, fl, ws, n_pad, k, nblk, n,
                                           update_tiles(k, kw, nblk, UPD_REST), st))
      return e;
    k += kw;
  }
  return SG_OK;
}

// Two streams: the rest of each group's update runs on the caller's update
// stream with two workgroups per CU instead of sharing a launch (and its
// 135 KB of LDS per workgroup) with the panel.  The two caller events order
// the streams: ev_panel once the panels a rest update reads are done,
// ev_rest after each rest update.  Same groups as the one-stream form, so
// the same result bit for bit.
struct SideStream {
  hipStream_t s;
  hipEvent_t ev_panel, ev_rest;
};

template <int R>
sg_status run_factor_split(const FactorLayers& fl, float* ws, int64_t n_pad, int nblk, int64_t n,
                           hipStream_t st, const SideStream* ss) {
  constexpr int parts = NB / R;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(panel_kernel<R>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PanelLds)) != hipSuccess)
    return set_error(SG_ERR_HIP, "hipFuncSetAttribute(panel kernel) failed");
  const auto api = [](hipError_t r, const char* what) -> sg_status {
    return r == hipSuccess ? SG_OK : set_error(SG_ERR_HIP, "factor: %s failed", what);
  };
  const dim3 pgrid((unsigned)(fl.nl * nblk * parts)), blk(256);
  // Caller's stream: panel 0; per group (after the previous group's rest
  // update, which covers the next block columns) the next-column updates,
  // the group's other panels, and the next panel.  Update stream: the rest
  // of the group's update, once its panels are done, beside the next panel.
  hipLaunchKernelGGL(panel_kernel<R>, pgrid, blk, sizeof(PanelLds), st, fl, ws, n_pad, 0, nblk, n);
  if (sg_status e = check_launch("factor panel")) return e;
  bool pending = false;  // a rest update was enqueued on the update stream
  for (int k = 0; k + 1 < nblk;) {
    if (pending)
      if (sg_status e = api(hipStreamWaitEvent(st, ss->ev_rest, 0), "stream wait")) return e;
    const int kw = std::min(KWMAX, nblk - 1 - k);
    for (int j = 1; j < kw; ++j) {
      if (sg_status e = launch_col_update(j, fl, ws, n_pad, k, nblk, st)) return e;
      hipLaunchKernelGGL(panel_kernel<R>, pgrid, blk, sizeof(PanelLds), st, fl, ws, n_pad, k + j, nblk, n);
      if (sg_status e = check_launch("factor panel")) return e;
    }
    if (sg_status e = api(hipEventRecord(ss->ev_panel, st), "event record")) return e;
    if (sg_status e = launch_col_update(kw, fl, ws, n_pad, k, nblk, st)) return e;
    const int64_t rest = update_tiles(k, kw, nblk, UPD_REST);
    if (rest > 0) {
      if (sg_status e = api(hipStreamWaitEvent(ss->s, ss->ev_panel, 0), "stream wait")) return e;
      if (sg_status e = launch_rest_update(kw, fl, ws, n_pad, k, nblk, rest, ss->s)) return e;
      if (sg_status e = api(hipEventRecord(ss->ev_rest, ss->s), "event record")) return e;
      pending = true;
    } else {
      pending = false;
    }
    hipLaunchKernelGGL(panel_kernel<R>, pgrid, blk, sizeof(PanelLds), st, fl, ws, n_pad, k + kw, nblk, n);
    if (sg_status e = check_launch("factor panel")) return e;
    k += kw;
  }
  // join: the caller's stream waits for the last trailing update
  if (pending)
    if (sg_status e = api(hipStreamWaitEvent(st, ss->ev_rest, 0), "stream wait")) return e;
  return SG_OK;
}

// ---- flip out: U[i][j] = Y[n-1-j][n-1-i] (i <= j), 0 below ------------------
__global__ __launch_bounds__(256) void finalize_kernel(const FactorLayers fl, const float* ws, int64_t n,
                                                       int64_t n_pad) {
  const int L = blockIdx.z;
  const float* __restrict__ Y = ws + L * fl.ls + n_pad * n_pad;
  float* __restrict__ U = fl.Hinv[L];
  __shared__ float tile[64][65];
  const int64_t I0 = blockIdx.y * 64, J0 = blockIdx.x * 64;
  const int c = threadIdx.x & 63, r0 = threadIdx.x >> 6;
  if (I0 > J0 + 63) {  // entirely below the diagonal
    for (int rr = r0; rr < 64; rr += 4) {
      const int64_t i = I0 + rr, j = J0 + c;
      if (i < n && j < n) U[i * n + j] = 0.f;
    }
    return;
  }
  // source rows a = n-1-J0-rr (rr = 0..63), columns b = n-1-I0-cc
  for (int rr = r0; rr < 64; rr += 4) {
    const int64_t a = n - 1 - (J0 + rr);
    const int64_t bcol = n - 1 - (I0 + c);
    float v = 0.f;
    if (a >= 0 && bcol >= 0) v = Y[a * n_pad + bcol];
    tile[rr][c] = v;  // tile[jj][ii] = Y[n-1-(J0+jj)][n-1-(I0+ii)]
  }
  __syncthreads();
  for (int rr = r0; rr < 64; rr += 4) {
    const int64_t i = I0 + rr, j = J0 + c;
    if (i < n && j < n) U[i * n + j] = (i <= j) ? tile[c][rr] : 0.f;
  }
}

}  // namespace

size_t factor_ws_bytes(int64_t n) {
  const int64_t n_pad = round_up(n, NB);
  return 2 * (size_t)n_pad * n_pad * sizeof(float) + 256;
}

namespace {

sg_status prepare_layers(const FactorLayers& fl, int64_t n, double damp, void* ws_v, hipStream_t st,
                         hipStream_t side, hipEvent_t ev_a, hipEvent_t ev_b) {
  const int64_t n_pad = round_up(n, NB);
  const int nblk = (int)(n_pad / NB);
  float* ws = static_cast<float*>(ws_v);

  hipLaunchKernelGGL(damp_lambda_kernel, dim3((unsigned)fl.nl), dim3(1024), 0, st, fl, ws, n, n_pad, damp);
  if (sg_status e = check_launch("damping")) return e;
  const unsigned t64 = (unsigned)(n_pad / 64);
  hipLaunchKernelGGL(flip_init_kernel, dim3(t64, t64, (unsigned)fl.nl), dim3(256), 0, st, fl, ws, n, n_pad);
  if (sg_status e = check_launch("flip/init")) return e;
  // Up to n = 4096 the panel chain sets the time: the panel takes four
  // workgroups per block (128 of the 256 CUs) and shares one launch with the
  // rest of the previous step's update, behind which its workgroups are
  // dispatched first (1.63 ms at n = 4096 against 1.98 ms on two streams,
  // where the update's workgroups delay the panel's).  At larger n the
  // trailing update sets the time: one panel workgroup per block, and the
  // update on its own stream at two workgroups per CU (n = 28672: 150 ms
  // against 182 ms in the shared launch).  Without a caller update stream
  // the single-stream fused form serves every n.  Several layers share each
  // launch (their panels first), so the latency-bound steps of one fill the
  // CUs the others leave idle.
  sg_status e;
  if (nblk * 8 <= kNumCU) {
    e = run_factor_fused<32, false>(fl, ws, n_pad, nblk, n, st);
  } else if (side != nullptr) {
    const SideStream ss{side, ev_a, ev_b};
    e = run_factor_split<128>(fl, ws, n_pad, nblk, n, st, &ss);
  } else {
    e = run_factor_fused<128, true>(fl, ws, n_pad, nblk, n, st);
  }
  if (e != SG_OK) return e;
  const unsigned tn = (unsigned)ceil_div(n, 64);
  hipLaunchKernelGGL(finalize_kernel, dim3(tn, tn, (unsigned)fl.nl), dim3(256), 0, st, fl, ws, n, n_pad);
  return check_launch("factor finalize");
}

}  // namespace

sg_status launch_prepare_hinv(float* Hinv, const float* H, int64_t n, double damp, int32_t* info,
                              void* ws, hipStream_t st, hipStream_t side, hipEvent_t ev_a,
                              hipEvent_t ev_b) {
  return launch_prepare_hinv_batched(&Hinv, &H, 1, n, damp, info, ws, st, side, ev_a, ev_b);
}

sg_status launch_prepare_hinv_batched(float* const* Hinv, const float* const* H, int nl, int64_t n,
                                      double damp, int32_t* info, void* ws, hipStream_t st,
                                      hipStream_t side, hipEvent_t ev_a, hipEvent_t ev_b) {
  FactorLayers fl{};
  fl.nl = nl;
  fl.ls = (int64_t)(factor_ws_bytes(n) / sizeof(float));
  for (int L = 0; L < nl; ++L) {
    fl.H[L] = H[L];
    fl.Hinv[L] = Hinv[L];
    fl.info[L] = info + L;
  }
  return prepare_layers(fl, n, damp, ws, st, side, ev_a, ev_b);
}

}  // namespace sg
