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
//   update kernel (fp32 MFMA, K = 128):
//     A[l,m] -= L[l,k] L[m,k]^T   for k < m <= l                     (SYRK)
//     R[c,l] -= Y[c,k] L[l,k]^T   for c <= k < l                      (inverse)
// where R is the running right-hand side of L X = I, kept transposed in the
// upper block triangle of Y (R starts as I).
#include "gemm_f32.h"

#include <math.h>

namespace sg {
namespace {

constexpr int NB = kFactorNB;  // 128
constexpr int LKS = 129;       // row stride of the scalar L_kk tile
constexpr int LIS = 132;       // row stride of L_kk^{-1} (16-byte aligned rows)

// ---- damping --------------------------------------------------------------
__global__ __launch_bounds__(256) void damp_lambda_kernel(const float* __restrict__ H, int64_t n,
                                                          double damp, float* lam_out,
                                                          int32_t* info) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += (double)H[i * n + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
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
// Y = I on the upper block triangle.  64x64 tiles.
__global__ __launch_bounds__(256) void flip_init_kernel(const float* __restrict__ H, int64_t n,
                                                        int64_t n_pad,
                                                        const float* __restrict__ lam_p,
                                                        float* __restrict__ A,
                                                        float* __restrict__ Y) {
  const int64_t ti = blockIdx.y, tj = blockIdx.x;
  const float lam = *lam_p;
  const int c = threadIdx.x & 63;
  const int r0 = threadIdx.x >> 6;
  const int64_t j = tj * 64 + c;
  // block-triangle membership at the 128 granularity of the factorisation
  const bool lower = (ti / 2) >= (tj / 2);
  const bool upper = (ti / 2) <= (tj / 2);
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
    if (upper) Y[i * n_pad + j] = (i == j) ? 1.f : 0.f;
  }
}

// ---- panel ---------------------------------------------------------------
struct PanelLds {
  float Lk[NB * LKS];
  float Li[NB * LIS];
  float Ld[NB];
  float Pst[GT * GS];
  int fail;
};

__global__ __launch_bounds__(256) void panel_kernel(float* __restrict__ A, float* __restrict__ Y,
                                                    int64_t n_pad, int k, int64_t n,
                                                    int32_t* info) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  PanelLds& S = *reinterpret_cast<PanelLds*>(smem);
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int64_t k0 = (int64_t)k * NB;

  // 1. load A_kk (lower part is all that is used)
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e >> 7, c = e & 127;
    S.Lk[i * LKS + c] = (c <= i) ? A[(k0 + i) * n_pad + k0 + c] : 0.f;
  }
  if (tid == 0) S.fail = -1;
  __syncthreads();

  // 2. unblocked right-looking Cholesky of A_kk in LDS
  const int tx = tid & 63, ty = tid >> 6;
  for (int j = 0; j < NB; ++j) {
    const float d2 = S.Lk[j * LKS + j];
    const float d = sqrtf(d2);
    const float r = 1.f / d;
    if (tid == 0) {
      S.Ld[j] = d;
      if (S.fail < 0 && !(d2 > 0.f && isfinite(d2))) S.fail = j;
    }
    if (tid > j && tid < NB) S.Lk[tid * LKS + j] *= r;
    __syncthreads();
    for (int i = j + 1 + ty; i < NB; i += 4) {
      const float lij = S.Lk[i * LKS + j];
      for (int c = j + 1 + tx; c <= i; c += 64) S.Lk[i * LKS + c] -= lij * S.Lk[c * LKS + j];
    }
    __syncthreads();
  }
  if (b == 0 && tid == 0 && S.fail >= 0) {
    const int64_t p = k0 + S.fail;  // column in the flipped order
    if (p < n) atomicCAS(info, 0, (int32_t)(n - p));
  }

  // 3. Li = L_kk^{-1} by right-looking forward substitution of L X = I.
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e >> 7, c = e & 127;
    S.Li[i * LIS + c] = (i == c) ? 1.f : 0.f;
  }
  __syncthreads();
  for (int i = 0; i < NB; ++i) {
    const float rd = 1.f / S.Ld[i];
    if (tid <= i) S.Li[i * LIS + tid] *= rd;
    __syncthreads();
    for (int rr = i + 1 + ty; rr < NB; rr += 4) {
      const float lri = S.Lk[rr * LKS + i];
      for (int c = tx; c <= i; c += 64) S.Li[rr * LIS + c] -= lri * S.Li[i * LIS + c];
    }
    __syncthreads();
  }

  // 4. apply
  if (b == k) {
    // Y[k,k] = L_kk^{-T}
    for (int e = tid; e < NB * NB; e += 256) {
      const int i = e >> 7, c = e & 127;
      Y[(k0 + i) * n_pad + k0 + c] = S.Li[c * LIS + i];
    }
    return;
  }
  float* blk;
  if (b > k)
    blk = A + (int64_t)b * NB * n_pad + k0;  // L[l,k] = A[l,k] L_kk^{-T}
  else
    blk = Y + (int64_t)b * NB * n_pad + k0;  // Y[c,k] = R[c,k] L_kk^{-T}
  const int wave = tid >> 6, lane = tid & 63;
  TileAcc acc;
  tile_zero(acc);
  for (int kc = 0; kc < NB; kc += GBK) {
    stage_rows_f32(S.Pst, blk, n_pad, NB, kc, NB);
    __syncthreads();
    // Q rows = rows of Li (k contiguous), taken straight from the inverse tile
    const int prow = (wave >> 1) * 64 + (lane & 15);
    const int qrow = (wave & 1) * 64 + (lane & 15);
#pragma unroll
    for (int g = 0; g < GBK / 16; ++g) {
      const int kl = g * 16 + (lane >> 4) * 4;
      floatx4 p[4], q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = *reinterpret_cast<const floatx4*>(S.Pst + (prow + i * 16) * GS + kl);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        q[jj] = *reinterpret_cast<const floatx4*>(S.Li + (qrow + jj * 16) * LIS + kc + kl);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc.v[i][jj] =
                __builtin_amdgcn_mfma_f32_16x16x4f32(p[i][e], q[jj][e], acc.v[i][jj], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        blk[(int64_t)tile_row(wave, lane, i, v) * n_pad + tile_col(wave, lane, jj)] = acc.v[i][jj][v];
}

// ---- trailing update ------------------------------------------------------
__device__ inline int64_t isqrt_floor(int64_t x) {
  int64_t r = (int64_t)sqrt((double)x);
  while (r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r;
}

__global__ __launch_bounds__(256) void update_kernel(float* __restrict__ A, float* __restrict__ Y,
                                                     int64_t n_pad, int k, int nblk) {
  __shared__ __attribute__((aligned(16))) float Pl[GT * GS];
  __shared__ __attribute__((aligned(16))) float Ql[GT * GS];
  const int64_t t = nblk - k - 1;  // trailing block count
  const int64_t nsyrk = t * (t + 1) / 2;
  int64_t idx = blockIdx.x;
  float *C;
  const float *P, *Q;
  if (idx < nsyrk) {
    // lower-triangle tile (l, m) of the trailing matrix, m <= l
    int64_t l = (isqrt_floor(8 * idx + 1) - 1) / 2;
    while ((l + 1) * (l + 2) / 2 <= idx) ++l;
    while (l * (l + 1) / 2 > idx) --l;
    const int64_t m = idx - l * (l + 1) / 2;
    const int64_t lb = k + 1 + l, mb = k + 1 + m;
    C = A + lb * NB * n_pad + mb * NB;
    P = A + lb * NB * n_pad + (int64_t)k * NB;
    Q = A + mb * NB * n_pad + (int64_t)k * NB;
  } else {
    idx -= nsyrk;
    const int64_t c = idx % (k + 1);
    const int64_t lb = k + 1 + idx / (k + 1);
    C = Y + c * NB * n_pad + lb * NB;
    P = Y + c * NB * n_pad + (int64_t)k * NB;
    Q = A + lb * NB * n_pad + (int64_t)k * NB;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  TileAcc acc;
  tile_zero(acc);
  for (int kc = 0; kc < NB; kc += GBK) {
    stage_rows_f32(Pl, P, n_pad, NB, kc, NB);
    stage_rows_f32(Ql, Q, n_pad, NB, kc, NB);
    __syncthreads();
    tile_mma_chunk(acc, Pl, Ql, wave, lane);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float* dst = C + (int64_t)tile_row(wave, lane, i, v) * n_pad + tile_col(wave, lane, jj);
        *dst -= acc.v[i][jj][v];
      }
}

// ---- flip out: U[i][j] = Y[n-1-j][n-1-i] (i <= j), 0 below ------------------
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ Y, int64_t n,
                                                       int64_t n_pad, float* __restrict__ U) {
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

sg_status launch_prepare_hinv(float* Hinv, const float* H, int64_t n, double damp, int32_t* info,
                              void* ws, hipStream_t st) {
  const int64_t n_pad = round_up(n, NB);
  const int nblk = (int)(n_pad / NB);
  float* A = static_cast<float*>(ws);
  float* Y = A + n_pad * n_pad;
  float* lam = Y + n_pad * n_pad;

  static bool attr_done = false;
  if (!attr_done) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(panel_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(PanelLds)) != hipSuccess)
      return set_error(SG_ERR_HIP, "hipFuncSetAttribute(panel_kernel) failed");
    attr_done = true;
  }

  hipLaunchKernelGGL(damp_lambda_kernel, dim3(1), dim3(256), 0, st, H, n, damp, lam, info);
  if (sg_status e = check_launch("damping")) return e;
  const unsigned t64 = (unsigned)(n_pad / 64);
  hipLaunchKernelGGL(flip_init_kernel, dim3(t64, t64), dim3(256), 0, st, H, n, n_pad, lam, A, Y);
  if (sg_status e = check_launch("flip/init")) return e;
  for (int k = 0; k < nblk; ++k) {
    hipLaunchKernelGGL(panel_kernel, dim3(nblk), dim3(256), sizeof(PanelLds), st, A, Y, n_pad, k,
                       n, info);
    if (sg_status e = check_launch("factor panel")) return e;
    const int64_t t = nblk - k - 1;
    const int64_t tiles = t * (t + 1) / 2 + (int64_t)(k + 1) * t;
    if (tiles > 0) {
      hipLaunchKernelGGL(update_kernel, dim3((unsigned)tiles), dim3(256), 0, st, A, Y, n_pad, k,
                         nblk);
      if (sg_status e = check_launch("factor update")) return e;
    }
  }
  const unsigned tn = (unsigned)ceil_div(n, 64);
  hipLaunchKernelGGL(finalize_kernel, dim3(tn, tn), dim3(256), 0, st, Y, n, n_pad, Hinv);
  return check_launch("factor finalize");
}

}  // namespace sg
