// Column sweep of the SparseGPT layer solver: mask selection, OBS prune and
// compensate, lazy trailing update.
//
// "SparseGPT ... Pruned in One-Shot" review (devpress): section 8 (choose a
// weight, estimate its error from the inverse Hessian, set it to zero, update
// the other not-yet-pruned weights of its row), section 11 steps 4-5 (columns
// are processed in blocks; the given fraction is pruned and the rest updated);
// section 14.4 and "Sparse Fine-tuning ..." section 8.4 (N:M keeps N of every M
// consecutive weights).  With U the upper factor of H_d^{-1}, pruning column j
// of row r removes e = W[r,j] / U_jj and subtracts e * U[j, j:] from the row.
//
// Per column block [i1, i1 + w):
//   select   (unstructured only) exact k-th smallest 64-bit key
//            (bits(W^2 / U_cc^2) << 32 | r*n + c) over the whole m x w block,
//            by a 6-pass 11/11/10-bit radix select; each pass builds an LDS
//            histogram per workgroup, and the last workgroup to finish scans
//            the merged histogram and fixes the next digit.
//   sweep    16 lanes per row, lane q owning columns q, q+16, ..., q+112 of the
//            block in registers; the owner of column j broadcasts e to its
//            row with a DPP row_newbcast; the U block sits in LDS with its
//            strictly lower part zero, so every lane updates every slot right
//            of the block start without predication.  N:M groups are ranked at
//            their first column through a small per-row LDS scratch.
//   lazy     W[:, i2:] -= Err * U[i1:i2, i2:] on fp32 MFMA (K = w).
#include "gemm_f32.h"

#include <math.h>

#include <type_traits>

namespace sg {
namespace {

constexpr int SB = SG_MAX_BLOCKSIZE;  // 128
constexpr int SW_ROWS = 16;           // rows per sweep workgroup
constexpr int SEL_EPT = 16;           // keys per thread per select pass

enum { MODE_THRESH = 0, MODE_NM = 1, MODE_FORCED = 2 };

struct SelState {
  unsigned long long prefix;
  unsigned long long thresh;
  long long krem;
  unsigned done;  // 0 searching, 1 thresh valid, 2 none selected, 3 all selected
  unsigned counter;
  unsigned hist[kSelBins];
};

__device__ inline float saliency(float w, float ucc) {
  const float q = w / ucc;
  return q * q;
}

__device__ inline unsigned long long sal_key(float w, float ucc, uint32_t lin) {
  return ((unsigned long long)__float_as_uint(saliency(w, ucc)) << 32) | lin;
}

__global__ void convert_kernel(float* __restrict__ out, const void* __restrict__ W, int dtype,
                               int64_t m, int64_t n, int64_t ldw) {
  const int64_t total = m * n;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / n, c = e - r * n;
    float v;
    if (dtype == SG_BF16)
      v = bf16_to_f32(static_cast<const uint16_t*>(W)[r * ldw + c]);
    else
      v = static_cast<const float*>(W)[r * ldw + c];
    out[e] = v;
  }
}

__global__ void sel_init_kernel(SelState* st, long long k, long long total) {
  for (int b = threadIdx.x; b < kSelBins; b += blockDim.x) st->hist[b] = 0u;
  if (threadIdx.x == 0) {
    st->prefix = 0ull;
    st->thresh = 0ull;
    st->krem = k;
    st->counter = 0u;
    st->done = (k <= 0) ? 2u : (k >= total ? 3u : 0u);
  }
}

__global__ __launch_bounds__(256) void sel_pass_kernel(SelState* st, const float* __restrict__ W,
                                                       const float* __restrict__ U, int64_t m,
                                                       int64_t n, int64_t i1, int w, int shift,
                                                       int width) {
  __shared__ unsigned h[kSelBins];
  __shared__ unsigned scan[256];
  __shared__ int s_last;
  if (st->done != 0u) return;
  const int tid = threadIdx.x;
  for (int b = tid; b < kSelBins; b += 256) h[b] = 0u;
  __syncthreads();
  const unsigned long long prefix = st->prefix;
  const int hi = shift + width;
  const unsigned dmask = (1u << width) - 1u;
  const int64_t total = m * (int64_t)w;
  const int64_t base = (int64_t)blockIdx.x * 256 * SEL_EPT;
  for (int u = 0; u < SEL_EPT; ++u) {
    const int64_t e = base + (int64_t)u * 256 + tid;
    if (e >= total) break;
    const int64_t r = e / w;
    const int c = (int)(e - r * w);
    const int64_t col = i1 + c;
    const unsigned long long key = sal_key(W[r * n + col], U[col * n + col], (uint32_t)(r * n + col));
    if (hi >= 64 || (key >> hi) == (prefix >> hi))
      atomicAdd(&h[(unsigned)(key >> shift) & dmask], 1u);
  }
  __syncthreads();
  for (int b = tid; b < kSelBins; b += 256)
    if (h[b]) atomicAdd(&st->hist[b], h[b]);
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&st->counter, 1u) == gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // Last workgroup: locate the digit holding the krem-th smallest key.
  const int per = kSelBins / 256;
  unsigned local = 0;
  for (int i = 0; i < per; ++i) {
    const unsigned v = __hip_atomic_load(&st->hist[tid * per + i], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    h[tid * per + i] = v;
    local += v;
  }
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
    const unsigned v = (tid >= off) ? scan[tid - off] : 0u;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const long long krem = st->krem;
  const unsigned long long before = (tid == 0) ? 0ull : scan[tid - 1];
  if ((long long)before < krem && krem <= (long long)scan[tid]) {
    unsigned long long cum = before;
    for (int i = 0; i < per; ++i) {
      const unsigned cnt = h[tid * per + i];
      if ((long long)(cum + cnt) >= krem) {
        const unsigned d = (unsigned)(tid * per + i);
        const unsigned long long np = prefix | ((unsigned long long)d << shift);
        const long long nk = krem - (long long)cum;
        st->prefix = np;
        st->krem = nk;
        if ((long long)cnt == nk) {
          st->thresh = np | ((shift > 0) ? ((1ull << shift) - 1ull) : 0ull);
          st->done = 1u;
        } else if (shift == 0) {
          st->thresh = np;
          st->done = 1u;
        }
        break;
      }
      cum += cnt;
    }
  }
  __syncthreads();
  for (int b = tid; b < kSelBins; b += 256) st->hist[b] = 0u;
  if (tid == 0) st->counter = 0u;
}

template <int L>
__device__ inline float bcast16_c(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + L, 0xF, 0xF, false));
}

struct SweepLds {
  float Ub[SB * SB];
  float Rd[SB];
  float Sc[SW_ROWS * SB];
};

template <int J, int END, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (J < END) {
    f(std::integral_constant<int, J>{});
    static_for<J + 1, END>(f);
  }
}

// Rank of key (my, me) among the group's keys sal[0..cnt) -- lexicographic
// (saliency, position), so equal saliencies prune the lower column first.
__device__ __forceinline__ int group_rank(const float* sal, int cnt, float my, int me) {
  int rank = 0;
  for (int t = 0; t < cnt; ++t) {
    const float o = sal[t];
    rank += (o < my || (o == my && t < me)) ? 1 : 0;
  }
  return rank;
}

__global__ __launch_bounds__(256) void sweep_kernel(float* __restrict__ W, uint8_t* __restrict__ mask_out,
                                                    float* __restrict__ Err, const float* __restrict__ U,
                                                    const uint8_t* __restrict__ mask_in,
                                                    const SelState* __restrict__ st, int64_t m,
                                                    int64_t n, int64_t i1, int w, int mode, int nkeep,
                                                    int mgroup) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SweepLds& S = *reinterpret_cast<SweepLds*>(smem);
  const int tid = threadIdx.x;
  const int q = tid & 15;
  const int rl = tid >> 4;
  const int64_t r = (int64_t)blockIdx.x * SW_ROWS + rl;
  const bool rv = r < m;

  for (int e = tid; e < SB * SB; e += 256) {
    const int j = e >> 7, c = e & (SB - 1);
    S.Ub[e] = (j < w && c < w && c >= j) ? U[(i1 + j) * n + i1 + c] : 0.f;
  }
  if (tid < SB) S.Rd[tid] = (tid < w) ? 1.f / U[(i1 + tid) * n + i1 + tid] : 0.f;
  float Wv[8], E[8];
  bool P[8];
  const int64_t rowoff = r * n + i1;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c = q + 16 * s;
    Wv[s] = (rv && c < w) ? W[rowoff + c] : 0.f;
    E[s] = 0.f;
    P[s] = false;
  }
  __syncthreads();

  if (mode == MODE_FORCED) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = q + 16 * s;
      P[s] = rv && c < w && mask_in[rowoff + c] != 0;
    }
  } else if (mode == MODE_THRESH) {
    const unsigned done = st->done;
    const unsigned long long thr = st->thresh;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = q + 16 * s;
      if (rv && c < w) {
        const unsigned long long key = sal_key(Wv[s], S.Ub[c * SB + c], (uint32_t)(rowoff + c));
        P[s] = (done == 3u) || (done == 1u && key <= thr);
      }
    }
  }
  const bool nm_small = (mode == MODE_NM) && mgroup <= 16;
  const bool nm_large = (mode == MODE_NM) && mgroup > 16;
  float* sc = S.Sc + rl * SB;

  static_for<0, SB>([&](auto Jc) {
    constexpr int J = decltype(Jc)::value;
    constexpr int qJ = J & 15, sJ = J >> 4;
    if (J >= w) return;
    if (nm_small && (J % mgroup) == 0) {
      // the group is columns J..J+M-1 = lanes qJ..qJ+M-1 of slot sJ
      const int c = q + 16 * sJ;
      const float sal = saliency(Wv[sJ], S.Ub[c * SB + c]);
      sc[q] = sal;
      __syncthreads();
      if (q >= qJ && q < qJ + mgroup)
        P[sJ] = rv && group_rank(sc + qJ, mgroup, sal, q - qJ) < mgroup - nkeep;
      __syncthreads();
    }
    if constexpr (qJ == 0) {
      if (nm_large && (J % mgroup) == 0) {
#pragma unroll
        for (int s = sJ; s < 8; ++s) {
          const int c = q + 16 * s;
          if (c < J + mgroup) sc[c - J] = saliency(Wv[s], S.Ub[c * SB + c]);
        }
        __syncthreads();
#pragma unroll
        for (int s = sJ; s < 8; ++s) {
          const int c = q + 16 * s;
          if (c < J + mgroup)
            P[s] = rv && group_rank(sc, mgroup, sc[c - J], c - J) < mgroup - nkeep;
        }
        __syncthreads();
      }
    }
    const float eo = (q == qJ && P[sJ]) ? Wv[sJ] * S.Rd[J] : 0.f;
    const float e = bcast16_c<qJ>(eo);
#pragma unroll
    for (int s = sJ; s < 8; ++s) Wv[s] = fmaf(-e, S.Ub[J * SB + q + 16 * s], Wv[s]);
    if (q == qJ) {
      E[sJ] = eo;
      if (P[sJ]) Wv[sJ] = 0.f;
    }
  });

  if (rv) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = q + 16 * s;
      if (c < w) {
        W[rowoff + c] = P[s] ? 0.f : Wv[s];
        if (mask_out) mask_out[rowoff + c] = P[s] ? 1 : 0;
        Err[r * SB + c] = E[s];
      }
    }
  }
}

// W[:, i2:] -= Err[:, 0:w] * U[i1:i2, i2:]
__global__ __launch_bounds__(256) void lazy_kernel(float* __restrict__ W, const float* __restrict__ Err,
                                                   const float* __restrict__ U, int64_t m, int64_t n,
                                                   int64_t i1, int w) {
  __shared__ __attribute__((aligned(16))) float Pl[GT * GS];
  __shared__ __attribute__((aligned(16))) float Ql[GT * GS];
  const int64_t i2 = i1 + w;
  const int64_t r0 = (int64_t)blockIdx.y * GT;
  const int64_t c0 = i2 + (int64_t)blockIdx.x * GT;
  const int rows = (int)min<int64_t>(GT, m - r0);
  const int cols = (int)min<int64_t>(GT, n - c0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  TileAcc acc;
  tile_zero(acc);
  for (int kc = 0; kc < w; kc += GBK) {
    stage_rows_f32(Pl, Err + r0 * SB, SB, rows, kc, w);
    stage_cols_f32(Ql, U + i1 * n + c0, n, cols, kc, w);
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
        const int rr = tile_row(wave, lane, i, v), cc = tile_col(wave, lane, jj);
        if (rr < rows && cc < cols) W[(r0 + rr) * n + c0 + cc] -= acc.v[i][jj][v];
      }
}

}  // namespace

size_t prune_ws_bytes(int64_t m, int64_t n, int blocksize) {
  (void)n;
  (void)blocksize;
  return round_up(sizeof(SelState), 256) + round_up((size_t)m * SB * sizeof(float), 256);
}

sg_status launch_prune(const PruneArgs& a, void* ws, hipStream_t st) {
  SelState* sel = static_cast<SelState*>(ws);
  float* Err = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up(sizeof(SelState), 256));
  const int64_t m = a.m, n = a.n;

  if (!(a.w_dtype == SG_F32 && static_cast<const void*>(a.W_out) == a.W)) {
    const int64_t total = m * n;
    const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(total, 256), 65536);
    hipLaunchKernelGGL(convert_kernel, dim3(grid), dim3(256), 0, st, a.W_out, a.W, a.w_dtype, m,
                       n, a.ldw);
    if (sg_status e = check_launch("prune convert")) return e;
  }
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(sweep_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)sizeof(SweepLds)) != hipSuccess)
    return set_error(SG_ERR_HIP, "hipFuncSetAttribute(sweep_kernel) failed");

  const int mode = a.mask_in ? MODE_FORCED : (a.kind == SG_NM ? MODE_NM : MODE_THRESH);
  const int B = a.blocksize;
  for (int64_t i1 = 0; i1 < n; i1 += B) {
    const int w = (int)std::min<int64_t>(B, n - i1);
    if (mode == MODE_THRESH) {
      const long long total = (long long)m * w;
      const long long k = (long long)floor(a.sparsity * (double)m * (double)w);
      hipLaunchKernelGGL(sel_init_kernel, dim3(1), dim3(256), 0, st, sel, k, total);
      if (sg_status e = check_launch("select init")) return e;
      const unsigned g = (unsigned)ceil_div(total, 256 * SEL_EPT);
      static const int shifts[6] = {53, 42, 32, 21, 10, 0};
      static const int widths[6] = {11, 11, 10, 11, 11, 10};
      for (int p = 0; p < 6; ++p) {
        hipLaunchKernelGGL(sel_pass_kernel, dim3(g), dim3(256), 0, st, sel, a.W_out, a.U, m, n, i1,
                           w, shifts[p], widths[p]);
        if (sg_status e = check_launch("select pass")) return e;
      }
    }
    hipLaunchKernelGGL(sweep_kernel, dim3((unsigned)ceil_div(m, SW_ROWS)), dim3(256),
                       sizeof(SweepLds), st, a.W_out, a.mask_out, Err, a.U, a.mask_in, sel, m, n,
                       i1, w, mode, a.n_keep, a.m_group);
    if (sg_status e = check_launch("prune sweep")) return e;
    const int64_t i2 = i1 + w;
    if (i2 < n) {
      dim3 grid((unsigned)ceil_div(n - i2, GT), (unsigned)ceil_div(m, GT));
      hipLaunchKernelGGL(lazy_kernel, grid, dim3(256), 0, st, a.W_out, Err, a.U, m, n, i1, w);
      if (sg_status e = check_launch("prune lazy")) return e;
    }
  }
  return SG_OK;
}

}  // namespace sg
