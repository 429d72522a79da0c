// Reconstruction error ||(W - W_hat) Xc^T||_F^2 of one calibration chunk.
//
// "SparseGPT ... Pruned in One-Shot" review (devpress), section 6: the layer
// objective is to keep W_hat X as close as possible to W X.  With token-major
// Xc[t, c], Y[r][t] = sum_c (W - W_hat)[r][c] Xc[t][c] is an NT contraction
// over the input channels; it runs on fp32 MFMA in 128x128 (rows x tokens)
// tiles, each tile squares and sums its outputs, and a single workgroup adds
// the per-tile partials in tile order in fp64 (reproducible).
#include "gemm_f32.h"

namespace sg {
namespace {

__device__ inline float load_elem(const void* p, int dtype, int64_t idx) {
  if (dtype == SG_BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[idx]);
  return static_cast<const float*>(p)[idx];
}

// P rows: D[r][k] = W[r][k] - W_hat[r][k]
struct DiffRows {
  const void* W;
  int wdt;
  int64_t ldw;
  const float* Wh;
  int64_t n;
  int rows;
  float w[GT / 8], h[GT / 8];
  __device__ inline void load(int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const int64_t k = k0 + kk;
    const int64_t kc = k < n ? k : n - 1;
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      const int rc = r < rows ? r : rows - 1;
      w[rr] = load_elem(W, wdt, (int64_t)rc * ldw + kc);
      h[rr] = Wh[(int64_t)rc * n + kc];
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const bool kok = k0 + kk < n;
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      lds[r * GS + kk] = (r < rows && kok) ? w[rr] - h[rr] : 0.f;
    }
  }
};

// Q rows: the token-major activations X[t][k]
struct XRows {
  const void* X;
  int xdt;
  int64_t ldx;
  int64_t n;
  int rows;
  float v[GT / 8];
  __device__ inline void load(int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const int64_t k = k0 + kk;
    const int64_t kc = k < n ? k : n - 1;
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      const int rc = r < rows ? r : rows - 1;
      v[rr] = load_elem(X, xdt, (int64_t)rc * ldx + kc);
    }
  }
  __device__ inline void store(float* lds, int64_t k0) {
    const int kk = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const bool kok = k0 + kk < n;
#pragma unroll
    for (int rr = 0; rr < GT / 8; ++rr) {
      const int r = r0 + rr * 8;
      lds[r * GS + kk] = (r < rows && kok) ? v[rr] : 0.f;
    }
  }
};

__global__ __launch_bounds__(256) void recon_tile_kernel(const void* __restrict__ W, int wdt,
                                                         int64_t ldw, const float* __restrict__ Wh,
                                                         int64_t m, int64_t n,
                                                         const void* __restrict__ X, int xdt,
                                                         int64_t T, int64_t ldx,
                                                         double* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float lds[4 * GBUF];
  __shared__ double red[4];
  const int64_t t0 = (int64_t)blockIdx.x * GT;
  const int64_t r0 = (int64_t)blockIdx.y * GT;
  const int rows = (int)min<int64_t>(GT, m - r0);
  const int toks = (int)min<int64_t>(GT, T - t0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t wsz = wdt == SG_BF16 ? 2 : 4, xsz = xdt == SG_BF16 ? 2 : 4;
  DiffRows pl{static_cast<const char*>(W) + r0 * ldw * wsz, wdt, ldw, Wh + r0 * n, n, rows};
  XRows ql{static_cast<const char*>(X) + t0 * ldx * xsz, xdt, ldx, n, toks};
  TileAcc acc;
  tile_zero(acc);
  tile_gemm_pipelined(acc, pl, ql, n, lds);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float y = acc.v[i][jj][v];
        s += (double)y * (double)y;
      }
  for (int off = 32; off > 0; off >>= 1) s += __shfl_down(s, off, 64);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ __launch_bounds__(256) void recon_reduce_kernel(const double* __restrict__ partial,
                                                           int64_t cnt, double* err, int accumulate) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < cnt; i += 256) s += partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *err = (accumulate ? *err : 0.0) + red[0];
}

}  // namespace

size_t recon_ws_bytes(int64_t m, int64_t T) {
  return round_up((size_t)ceil_div(m, GT) * ceil_div(T, GT) * sizeof(double), 256);
}

sg_status launch_recon(double* err, int accumulate, const void* W, int w_dtype, int64_t ldw,
                       const float* W_hat, int64_t m, int64_t n, const void* X, int x_dtype,
                       int64_t T, int64_t ldx, void* ws, hipStream_t st) {
  double* partial = static_cast<double*>(ws);
  dim3 grid((unsigned)ceil_div(T, GT), (unsigned)ceil_div(m, GT));
  hipLaunchKernelGGL(recon_tile_kernel, grid, dim3(256), 0, st, W, w_dtype, ldw, W_hat, m, n, X,
                     x_dtype, T, ldx, partial);
  if (sg_status e = check_launch("recon tiles")) return e;
  hipLaunchKernelGGL(recon_reduce_kernel, dim3(1), dim3(256), 0, st, partial,
                     (int64_t)grid.x * grid.y, err, accumulate);
  return check_launch("recon reduce");
}

}  // namespace sg
