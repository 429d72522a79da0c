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

#include <hip/hip_cooperative_groups.h>

#include <math.h>

#include <type_traits>
#include <utility>

namespace sg {
namespace {

constexpr int SB = SG_MAX_BLOCKSIZE;  // 128
constexpr int SW_ROWS = 16;           // rows per sweep workgroup

enum { MODE_THRESH = 0, MODE_NM = 1, MODE_FORCED = 2 };

struct SelState {
  unsigned long long thresh;
  unsigned done;  // 1 thresh valid, 2 none selected, 3 all selected
  unsigned pad;
  unsigned hist[3][kSelBins];  // per-pass merged histograms, used round-robin
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

__global__ void sel_clear_kernel(SelState* st) {
  for (int b = threadIdx.x; b < 3 * kSelBins; b += blockDim.x) (&st->hist[0][0])[b] = 0u;
}

// Exact k-th smallest 64-bit key of the m x w block by radix select, all
// passes in one cooperative launch.  Every thread computes the keys of its
// (at most SEL_KPT) elements once and keeps them in registers.  Each pass
// histograms one digit of the keys that still match the prefix fixed so far
// (eight lane-interleaved LDS sub-histograms against atomic contention on
// hot bins, merged into a global one); after a grid-wide sync every
// workgroup scans the merged histogram itself and fixes the same digit.
// hist[p % 3] is used by pass p; workgroup 0 clears the next pass's buffer
// during the current pass (its readers finished two syncs earlier).  hist[0]
// must be zero on entry; the sweep kernel that follows re-clears all three.
constexpr int SEL_KPT = 32;   // keys per thread held in registers
constexpr int SEL_SUB = 8;    // LDS sub-histograms

__global__ __launch_bounds__(256) void select_kernel(SelState* st, const float* __restrict__ W,
                                                    const float* __restrict__ U, int64_t m,
                                                    int64_t n, int64_t i1, int w, long long k) {
  namespace cg = cooperative_groups;
  cg::grid_group grid = cg::this_grid();
  __shared__ unsigned h[SEL_SUB][kSelBins];
  __shared__ unsigned wsum[4];
  __shared__ unsigned long long s_prefix;
  __shared__ long long s_krem;
  __shared__ unsigned s_done;
  __shared__ unsigned long long s_thresh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long total = m * (long long)w;
  if (tid == 0) {
    s_prefix = 0ull;
    s_krem = k;
    s_done = (k <= 0) ? 2u : (k >= total ? 3u : 0u);
    s_thresh = 0ull;
  }
  // keys of this thread: column c, rows rb + u * rstep (u < SEL_KPT)
  const int c = tid & 127;
  const int cc = c < w ? c : w - 1;
  const int64_t col = i1 + cc;
  const float ucc = U[col * n + col];
  const int64_t rstep = (int64_t)gridDim.x * 2;
  const int64_t rb = (int64_t)blockIdx.x * 2 + (tid >> 7);
  unsigned long long keys[SEL_KPT];
  {
    float wv[SEL_KPT];
#pragma unroll
    for (int u = 0; u < SEL_KPT; ++u) {
      const int64_t r = rb + u * rstep;
      wv[u] = W[(r < m ? r : m - 1) * n + col];
    }
#pragma unroll
    for (int u = 0; u < SEL_KPT; ++u) {
      const int64_t r = rb + u * rstep;
      // out-of-range slots get the largest key, which never matches a prefix
      keys[u] = (r < m && c < w) ? sal_key(wv[u], ucc, (uint32_t)(r * n + col)) : ~0ull;
    }
  }
  __syncthreads();
  static const int shifts[6] = {53, 42, 32, 21, 10, 0};
  static const int widths[6] = {11, 11, 10, 11, 11, 10};
  unsigned* hsub = h[lane & (SEL_SUB - 1)];
  for (int p = 0; p < 6; ++p) {
    if (s_done != 0u) break;  // uniform across the grid
    const int shift = shifts[p], width = widths[p];
    const int hi = shift + width;
    const unsigned dmask = (1u << width) - 1u;
    const unsigned long long prefix = s_prefix;
    unsigned* gh = st->hist[p % 3];
    if (blockIdx.x == 0)
      for (int b = tid; b < kSelBins; b += 256) st->hist[(p + 1) % 3][b] = 0u;
    for (int b = tid; b < SEL_SUB * kSelBins; b += 256) (&h[0][0])[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < SEL_KPT; ++u) {
      const unsigned long long key = keys[u];
      if (key != ~0ull && (hi >= 64 || (key >> hi) == (prefix >> hi)))
        atomicAdd(&hsub[(unsigned)(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    for (int b = tid; b < kSelBins; b += 256) {
      unsigned v = 0;
#pragma unroll
      for (int sh = 0; sh < SEL_SUB; ++sh) v += h[sh][b];
      if (v) atomicAdd(&gh[b], v);
    }
    grid.sync();
    // every workgroup: locate the digit holding the krem-th smallest key;
    // thread t owns bins 8t..8t+7, prefix sums by wave shuffles
    const int per = kSelBins / 256;
    unsigned cnt[per];
    unsigned local = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      cnt[i] = gh[tid * per + i];
      local += cnt[i];
    }
    unsigned incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned wbase = 0;
    for (int wv2 = 0; wv2 < wave; ++wv2) wbase += wsum[wv2];
    const long long krem = s_krem;
    const unsigned long long before = (unsigned long long)(wbase + incl - local);
    const unsigned long long after = (unsigned long long)(wbase + incl);
    __syncthreads();
    if ((long long)before < krem && krem <= (long long)after) {
      unsigned long long cum = before;
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const unsigned cn = cnt[i];
        if ((long long)cum < krem && (long long)(cum + cn) >= krem) {
          const unsigned d = (unsigned)(tid * per + i);
          const unsigned long long np = prefix | ((unsigned long long)d << shift);
          const long long nk = krem - (long long)cum;
          s_prefix = np;
          s_krem = nk;
          if ((long long)cn == nk || shift == 0) {
            // the bucket is taken whole: every key up to the end of its range
            s_thresh = np | ((shift > 0) ? ((1ull << shift) - 1ull) : 0ull);
            s_done = 1u;
          }
        }
        cum += cn;
      }
    }
    __syncthreads();
  }
  if (blockIdx.x == 0 && tid == 0) {
    st->done = s_done;
    st->thresh = s_thresh;
  }
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

struct SweepCtx {
  float* sc;       // per-row scratch of the N:M ranking
  const float* Ub; // U block in LDS
  const float* Rd; // reciprocal diagonal in LDS
  int q, w, mgroup, nkeep, sb;
  bool rv, nm_small;
};

// Column J = 16*sb + QJ of the in-block sweep.  Register slot s holds column
// q + 16*(sb + s) (the slots rotate down after every 16 columns), so the owner
// of column J is lane QJ, slot 0: QJ is a compile-time constant, making the
// DPP broadcast and every register index static.
template <int QJ, bool NM>
__device__ __forceinline__ void sweep_col(const SweepCtx& cx, float (&Wv)[8], float (&E)[8],
                                          bool (&P)[8]) {
  const int J = cx.sb * 16 + QJ;
  const int q = cx.q;
  if constexpr (NM) {
    if (J < cx.w && cx.nm_small && (J % cx.mgroup) == 0) {
      // the group is columns J..J+M-1 = lanes QJ..QJ+M-1 of slot 0
      const int c = q + 16 * cx.sb;
      const float sal = saliency(Wv[0], cx.Ub[c * SB + c]);
      cx.sc[q] = sal;
      __syncthreads();
      if (q >= QJ && q < QJ + cx.mgroup)
        P[0] = cx.rv && group_rank(cx.sc + QJ, cx.mgroup, sal, q - QJ) < cx.mgroup - cx.nkeep;
      __syncthreads();
    }
  }
  // Branch-free step (columns past the block are no-ops: P is false there and
  // the U block is zero), so 16 steps form one basic block and the scheduler
  // can issue the U-row reads of later steps early.
  const int Jr = J < SB ? J : SB - 1;
  const float rdj = cx.Rd[Jr];
  float u[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int as = s + cx.sb;  // absolute slot; past the block the U row is zero
    const float uv = cx.Ub[Jr * SB + q + 16 * (as < 8 ? as : 7)];
    u[s] = as < 8 ? uv : 0.f;
  }
  const bool own = (q == QJ) && (J < cx.w);
  const bool prune = own && P[0];
  const float eo = prune ? Wv[0] * rdj : 0.f;
  const float e = bcast16_c<QJ>(eo);
#pragma unroll
  for (int s = 0; s < 8; ++s) Wv[s] = fmaf(-e, u[s], Wv[s]);
  E[0] = own ? eo : E[0];
  Wv[0] = prune ? 0.f : Wv[0];
}

template <bool NM, int... Qs>
__device__ __forceinline__ void sweep_16(std::integer_sequence<int, Qs...>, const SweepCtx& cx,
                                         float (&Wv)[8], float (&E)[8], bool (&P)[8]) {
  (sweep_col<Qs, NM>(cx, Wv, E, P), ...);
}

template <int MODE>
__global__ __launch_bounds__(256) void sweep_kernel(float* __restrict__ W, uint8_t* __restrict__ mask_out,
                                                    float* __restrict__ Err, const float* __restrict__ U,
                                                    const uint8_t* __restrict__ mask_in,
                                                    const SelState* __restrict__ st, int64_t m,
                                                    int64_t n, int64_t i1, int w, int nkeep,
                                                    int mgroup) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SweepLds& S = *reinterpret_cast<SweepLds*>(smem);
  const int tid = threadIdx.x;
  const int q = tid & 15;
  const int rl = tid >> 4;
  const int64_t r = (int64_t)blockIdx.x * SW_ROWS + rl;
  const bool rv = r < m;

  {
    // U block: row j = tid/2, 64 columns per thread; all loads issued together
    // from clamped in-bounds addresses, out-of-block entries zeroed on store
    const int j = tid >> 1, c0 = (tid & 1) * 64;
    const int jc = j < w ? j : w - 1;
    const float* urow = U + (i1 + jc) * n + i1;
    float uv[64];
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      const int c = c0 + u;
      uv[u] = urow[c < w ? c : w - 1];
    }
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      const int c = c0 + u;
      S.Ub[j * SB + c] = (j < w && c < w && c >= j) ? uv[u] : 0.f;
    }
  }
  if (tid < SB) S.Rd[tid] = (tid < w) ? 1.f / U[(i1 + tid) * n + i1 + tid] : 0.f;
  if (MODE == MODE_THRESH && blockIdx.x == 0) {
    // leave the select histograms zeroed for the next block (the select
    // launch of this block has completed)
    SelState* sw = const_cast<SelState*>(st);
    for (int b = tid; b < 3 * kSelBins; b += 256) (&sw->hist[0][0])[b] = 0u;
  }
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

  if (MODE == MODE_FORCED) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = q + 16 * s;
      P[s] = rv && c < w && mask_in[rowoff + c] != 0;
    }
  } else if (MODE == MODE_THRESH) {
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

  SweepCtx cx;
  cx.sc = S.Sc + rl * SB;
  cx.Ub = S.Ub;
  cx.Rd = S.Rd;
  cx.q = q;
  cx.w = w;
  cx.mgroup = mgroup;
  cx.nkeep = nkeep;
  cx.rv = rv;
  cx.nm_small = (MODE == MODE_NM) && mgroup <= 16;
  const bool nm_large = (MODE == MODE_NM) && mgroup > 16;
  for (int sb = 0; sb < 8; ++sb) {
    if (sb * 16 >= w) break;
    cx.sb = sb;
    if (MODE == MODE_NM && nm_large && ((sb * 16) % mgroup) == 0) {
      // group of M >= 16 columns starting here: slots 0 .. M/16-1, all lanes
      const int J = sb * 16;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = q + 16 * (s + sb);
        if (s + sb < 8 && c < J + mgroup) cx.sc[c - J] = saliency(Wv[s], S.Ub[c * SB + c]);
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = q + 16 * (s + sb);
        if (s + sb < 8 && c < J + mgroup)
          P[s] = rv && group_rank(cx.sc, mgroup, cx.sc[c - J], c - J) < mgroup - nkeep;
      }
      __syncthreads();
    }
    sweep_16<MODE == MODE_NM>(std::make_integer_sequence<int, 16>{}, cx, Wv, E, P);
    // retire slot 0 (column q + 16*sb) and rotate the slots down
    const int c = q + 16 * sb;
    if (rv && c < w) {
      W[rowoff + c] = P[0] ? 0.f : Wv[0];
      if (mask_out) mask_out[rowoff + c] = P[0] ? 1 : 0;
      Err[r * SB + c] = E[0];
    }
#pragma unroll
    for (int s = 0; s < 7; ++s) {
      Wv[s] = Wv[s + 1];
      E[s] = E[s + 1];
      P[s] = P[s + 1];
    }
    Wv[7] = 0.f;
    E[7] = 0.f;
    P[7] = false;
  }
}

// W[:, i2:] -= Err[:, 0:w] * U[i1:i2, i2:]
__global__ __launch_bounds__(256) void lazy_kernel(float* __restrict__ W, const float* __restrict__ Err,
                                                   const float* __restrict__ U, int64_t m, int64_t n,
                                                   int64_t i1, int w) {
  __shared__ __attribute__((aligned(16))) float lds[4 * GBUF];
  const int64_t i2 = i1 + w;
  const int64_t r0 = (int64_t)blockIdx.y * GT;
  const int64_t c0 = i2 + (int64_t)blockIdx.x * GT;
  const int rows = (int)min<int64_t>(GT, m - r0);
  const int cols = (int)min<int64_t>(GT, n - c0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  RowsF32 pl{Err + r0 * SB, SB, rows, w, 1.f};
  ColsF32 ql{U + i1 * n + c0, n, cols, w};
  TileAcc acc;
  tile_zero(acc);
  tile_gemm_pipelined(acc, pl, ql, w, lds);
  tile_sub_from(W + r0 * n + c0, n, rows, cols, acc, lds);
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
  const void* sweep_fns[3] = {reinterpret_cast<const void*>(sweep_kernel<MODE_THRESH>),
                              reinterpret_cast<const void*>(sweep_kernel<MODE_NM>),
                              reinterpret_cast<const void*>(sweep_kernel<MODE_FORCED>)};
  for (const void* f : sweep_fns)
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(SweepLds)) !=
        hipSuccess)
      return set_error(SG_ERR_HIP, "hipFuncSetAttribute(sweep_kernel) failed");

  const int mode = a.mask_in ? MODE_FORCED : (a.kind == SG_NM ? MODE_NM : MODE_THRESH);
  const int B = a.blocksize;
  int64_t sel_grid_cap = 0;
  if (mode == MODE_THRESH) {
    int dev = 0, ncu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(select_kernel),
                                                     256, 0) != hipSuccess || per_cu < 1)
      return set_error(SG_ERR_HIP, "select kernel occupancy query failed");
    sel_grid_cap = (int64_t)ncu * per_cu;
    hipLaunchKernelGGL(sel_clear_kernel, dim3(1), dim3(256), 0, st, sel);
    if (sg_status e = check_launch("select clear")) return e;
  }
  for (int64_t i1 = 0; i1 < n; i1 += B) {
    const int w = (int)std::min<int64_t>(B, n - i1);
    if (mode == MODE_THRESH) {
      const long long k = (long long)floor(a.sparsity * (double)m * (double)w);
      const long long total = (long long)m * w;
      // enough workgroups that every thread holds at most SEL_KPT keys
      const int64_t need = ceil_div(m, (int64_t)2 * SEL_KPT);
      if (need > sel_grid_cap)
        return set_error(SG_ERR_UNSUPPORTED, "m=%lld too large for the single-launch select",
                         (long long)m);
      const unsigned g = (unsigned)std::max<int64_t>(1, need);
      void* args[] = {&sel, const_cast<float**>(&a.W_out), const_cast<float**>(&a.U),
                      const_cast<int64_t*>(&a.m), const_cast<int64_t*>(&a.n), &i1,
                      const_cast<int*>(&w), const_cast<long long*>(&k)};
      if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(select_kernel), dim3(g), dim3(256),
                                     args, 0, st) != hipSuccess)
        return set_error(SG_ERR_HIP, "cooperative launch of the select kernel failed");
      if (sg_status e = check_launch("select")) return e;
    }
    {
      const dim3 sg_grid((unsigned)ceil_div(m, SW_ROWS)), sg_block(256);
      const size_t shm = sizeof(SweepLds);
      if (mode == MODE_THRESH)
        hipLaunchKernelGGL(sweep_kernel<MODE_THRESH>, sg_grid, sg_block, shm, st, a.W_out, a.mask_out,
                           Err, a.U, a.mask_in, sel, m, n, i1, w, a.n_keep, a.m_group);
      else if (mode == MODE_NM)
        hipLaunchKernelGGL(sweep_kernel<MODE_NM>, sg_grid, sg_block, shm, st, a.W_out, a.mask_out, Err,
                           a.U, a.mask_in, sel, m, n, i1, w, a.n_keep, a.m_group);
      else
        hipLaunchKernelGGL(sweep_kernel<MODE_FORCED>, sg_grid, sg_block, shm, st, a.W_out, a.mask_out,
                           Err, a.U, a.mask_in, sel, m, n, i1, w, a.n_keep, a.m_group);
    }
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
