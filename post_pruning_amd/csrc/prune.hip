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
//   select   (block-global unstructured only) exact k-th smallest 64-bit key
//            (bits(W^2 / U_cc^2) << 32 | r*n + c) of each stacked matrix's
//            m x w block: two radix passes (11-bit digits) here, finished by
//            every sweep workgroup (sweep.h);
//   sweep    the in-block OBS prune and compensate of sweep.h, instantiated
//            in sweep_plain.hip, sweep_quant.hip and sweep_joint.hip; N:M and
//            per-row groups are ranked inside it;
//   lazy     W[:, i2:] -= Err * U[i1:i2, i2:] on fp32 MFMA, in two levels:
//            the rest of the 512-column group after each block (K = w), the
//            columns beyond the group after its last block (K = 512).
#include "gemm_x6.h"
#include "sweep.h"

#include <math.h>

#include <mutex>
#include <type_traits>
#include <utility>

namespace sg {
namespace {

// W (bf16 or fp32, row stride ldw) -> out (fp32, row stride n).  Each
// thread converts 8 consecutive columns of a row (blockIdx.x picks 2048
// columns, blockIdx.y strides over the rows): 16-byte accesses when every
// row of both matrices is 16-byte aligned (vec), element by element
// otherwise and in a row's last partial group.
__global__ __launch_bounds__(256) void convert_kernel(float* __restrict__ out, const void* __restrict__ W,
                                                      int dtype, int64_t m, int64_t n, int64_t ldw, int vec) {
  const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= n) return;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    float* o = out + r * n + c0;
    if (vec && c0 + 8 <= n) {
      if (dtype == SG_BF16) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + r * ldw + c0);
        floatx4 lo, hi;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          lo[2 * q] = __uint_as_float(x[q] << 16);
          lo[2 * q + 1] = __uint_as_float(x[q] & 0xffff0000u);
          hi[2 * q] = __uint_as_float(x[q + 2] << 16);
          hi[2 * q + 1] = __uint_as_float(x[q + 2] & 0xffff0000u);
        }
        *reinterpret_cast<floatx4*>(o) = lo;
        *reinterpret_cast<floatx4*>(o + 4) = hi;
      } else {
        const float* src = static_cast<const float*>(W) + r * ldw + c0;
        *reinterpret_cast<floatx4*>(o) = *reinterpret_cast<const floatx4*>(src);
        *reinterpret_cast<floatx4*>(o + 4) = *reinterpret_cast<const floatx4*>(src + 4);
      }
    } else {
      for (int e = 0; e < 8 && c0 + e < n; ++e)
        o[e] = dtype == SG_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(W)[r * ldw + c0 + e])
                                : static_cast<const float*>(W)[r * ldw + c0 + e];
    }
  }
}

__global__ void sel_clear_kernel(SelState* st) {  // one workgroup per segment
  sel_clear_set(st[blockIdx.x].set[0], threadIdx.x, blockDim.x);
  sel_clear_set(st[blockIdx.x].set[1], threadIdx.x, blockDim.x);
}
struct SelLds {
  unsigned h[SEL_SUB][kSelBins];
  unsigned long long stage[SEL_SORT];
  unsigned nstage;
  unsigned gbase;
  HistPick pick;
};

__global__ __launch_bounds__(256) void select_pass_kernel(SelState* st, int parity,
                                                         unsigned long long* cand,
                                                         const float* __restrict__ W, const Segs segs,
                                                         int64_t n, int64_t i1, int w, int pass) {
  // blockIdx.y = segment; its keys only, into its own histograms and list
  const int seg = blockIdx.y;
  if (segs.fixed[seg] != 0) return;  // whole workgroup: nothing to select
  const float* __restrict__ U = segs.U[seg];
  const long long k = segs.k[seg];
  SelSet* ss = &st[seg].set[parity];
  cand += segs.row0[seg] * SB;
  const int64_t rlo = segs.row0[seg], m = segs.row0[seg + 1];
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SelLds& L = *reinterpret_cast<SelLds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  // pass 0 counts every key (lane-interleaved sub-histograms against hot
  // bins); pass 1 only the few keys under the top digit (one histogram)
  const int nsub = pass == 0 ? SEL_SUB : 1;
  for (int b = tid; b < nsub * kSelBins; b += 256) (&L.h[0][0])[b] = 0u;
  if (tid == 0) L.nstage = 0u;
  // this thread's keys are requested first: their latency overlaps the scan
  // of the top-digit histogram
  const int shift = pass == 0 ? 53 : 42;
  const unsigned dmask = (1u << 11) - 1u;
  const int c = tid & 127;
  const int cc = c < w ? c : w - 1;
  const int64_t col = i1 + cc;
  const float ucol = U[col * n + col];
  const int64_t rstep = (int64_t)gridDim.x * 2;
  const int64_t rb = rlo + (int64_t)blockIdx.x * 2 + (tid >> 7);
  float wv[SEL_KPT];
#pragma unroll
  for (int u = 0; u < SEL_KPT; ++u) {
    const int64_t r = rb + u * rstep;
    wv[u] = W[(r < m ? r : m - 1) * n + col];
  }
  unsigned top = 0;
  if (pass == 1) {
    hist_locate(ss->hist0, k, L.pick);  // (includes a barrier)
    top = L.pick.digit;
  }
  const float rd = 1.f / ucol;
  __syncthreads();
  unsigned* hsub = L.h[pass == 0 ? (lane & (SEL_SUB - 1)) : 0];
#pragma unroll
  for (int u = 0; u < SEL_KPT; ++u) {
    const int64_t r = rb + u * rstep;
    if (r < m && c < w) {
      const unsigned long long key = sal_key(wv[u], rd, (uint32_t)(r * n + col));
      if (pass == 0 || (unsigned)(key >> 53) == top) {
        atomicAdd(&hsub[(unsigned)(key >> shift) & dmask], 1u);
        if (pass == 1) L.stage[atomicAdd(&L.nstage, 1u)] = key;
      }
    }
  }
  __syncthreads();
  unsigned* gh = pass == 0 ? ss->hist0 : ss->hist1;
  for (int b = tid; b < kSelBins; b += 256) {
    unsigned v = 0;
    for (int sh = 0; sh < nsub; ++sh) v += L.h[sh][b];
    if (v) atomicAdd(&gh[b], v);
  }
  if (pass == 1) {
    // this workgroup's gathered keys to the candidate list (one reservation)
    if (tid == 0) L.gbase = atomicAdd(&ss->ncand, L.nstage);
    __syncthreads();
    for (unsigned i = tid; i < L.nstage; i += 256) cand[L.gbase + i] = L.stage[i];
  }
}

// Per-row grid of the joint sparse + quantized sweep, from the row's original
// weights: lo = min(0, min w), hi = max(0, max w), scale = (hi - lo) / L
// (1 for an all-zero row), zero = round(-lo / scale).  One workgroup per row.
// scale and the zero point are formed in fp64 (lo and hi are exact): bf16
// rows often have hi = -lo, where -lo / scale sits on a half-way point and
// the rounding of fp32 intermediates would decide the zero point.
__global__ __launch_bounds__(256) void qgrid_kernel(const float* __restrict__ W, int64_t n, float L,
                                                    float* __restrict__ scale, float* __restrict__ zero) {
  __shared__ float red[2][4];
  const float* row = W + (int64_t)blockIdx.x * n;
  float lo = 0.f, hi = 0.f;
  for (int64_t c = threadIdx.x; c < n; c += 256) {
    const float x = row[c];
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = lo;
    red[1][threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    lo = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
    hi = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    const double s = hi > lo ? ((double)hi - (double)lo) / (double)L : 1.0;
    scale[blockIdx.x] = (float)s;
    zero[blockIdx.x] = (float)rint(-(double)lo / s);
  }
}

// Epilogue hook of the lazy update: the tiles that hold the next block's
// final values count their saliency keys' top digit into an LDS histogram
// (the first radix-select pass of that block, taken where the values are
// produced).  Same digit and same fp32 saliency as select_pass_kernel.
struct TopDigitHist {
  unsigned* lh;       // LDS [kSelBins]
  const float* lrd;   // LDS [T]: 1 / U_cc of the tile's columns
  int ncols;          // tile columns inside the next block
  __device__ void operator()(int, int c, float v) const {
    if (c < ncols) atomicAdd(&lh[__float_as_uint(saliency(v, lrd[c])) >> 21], 1u);
  }
};

// W[:, c_begin:c_end] -= E[:, 0:K] * U[k0:k0+K, c_begin:c_end]; E has row stride
// EGK.  The lazy update of the column sweep, in two levels: after each block
// its errors update the rest of the current group of columns (K = block
// width); after the last block of a group, the errors of the whole group
// update every column beyond it at once (K = group width).  blockIdx.z picks
// a row segment (its rows and its factor U).  With hist0 set, the tiles over
// the next block's first hist_w columns also add that block's top-digit
// histogram into hist0.

template <bool VEC, int T, bool SHORT = false>
__global__ __launch_bounds__(256, 2) void lazy_kernel(float* __restrict__ W, const float* __restrict__ E,
                                                      const Segs segs, int64_t n,
                                                      int64_t k0, int K, int64_t c_begin, int64_t c_end,
                                                      unsigned* __restrict__ hist0, int hist_w) {
  constexpr int LDSB = VEC ? (SHORT ? X6Lds<T>::SHORT : X6Lds<T>::SIZE) : 4 * T * GS * 4;
  __shared__ __attribute__((aligned(16))) unsigned char ldsb[LDSB];
  __shared__ unsigned lhist[kSelBins];
  __shared__ float lrd[T];
  float* lds = reinterpret_cast<float*>(ldsb);
  const int seg = blockIdx.z;
  const int64_t m = segs.row0[seg + 1];
  const int64_t r0 = segs.row0[seg] + (int64_t)blockIdx.y * T;
  if (r0 >= m) return;  // whole workgroup: past a shorter segment
  const float* __restrict__ U = segs.U[seg];
  const int64_t c0 = c_begin + (int64_t)blockIdx.x * T;
  const int rows = (int)min<int64_t>(T, m - r0);
  const int cols = (int)min<int64_t>(T, c_end - c0);
  float* C = W + r0 * n + c0;
  // tiles over the next block's columns [c_begin, c_begin + hist_w)
  const bool hist = hist0 != nullptr && (int64_t)blockIdx.x * T < hist_w;
  const TopDigitHist hk{lhist, lrd, (int)min<int64_t>(cols, hist_w - (int64_t)blockIdx.x * T)};
  // the tile's diagonal entries of U are requested now and stored to LDS
  // after the products (their latency hides behind them)
  float ucc = 1.f;
  if (hist) {
    for (int b = threadIdx.x; b < kSelBins; b += 256) lhist[b] = 0u;
    if (threadIdx.x < T) {
      const int64_t c = c0 + (threadIdx.x < cols ? threadIdx.x : 0);
      ucc = U[c * n + c];
    }
  }
  TileAccT<T> acc;
  tile_zero(acc);
  bool done = false;
  if constexpr (VEC && SHORT) {
    // one block's errors (K <= 128): the operands and the W tile are all
    // requested before the first product
    CTileV<T> ct;
    const bool cpre = CTileV<T>::ok(C, n, cols);
    if (cpre) ct.load(C, n, rows);
    RowsX6V<T> pl{E + r0 * EGK, EGK, rows, K};
    ColsX6T<T> ql{U + k0 * n + c0, n, cols, K};
    tile_gemm_x6_short<T, SB / GBK>(acc, pl, ql, K, ldsb);
    if (hist && threadIdx.x < T) lrd[threadIdx.x] = 1.f / ucc;
    if (cpre) {
      if (hist)
        tile_sub_pre(C, n, rows, ct, acc, lds, hk);
      else
        tile_sub_pre(C, n, rows, ct, acc, lds);
      done = true;
    }
  } else if constexpr (VEC) {
    // fp32-accurate products on bf16 MFMA (three-way split, six terms); full
    // tiles take loaders without the clamped path (fewer live registers)
    if (rows == T && cols == T && (K % GBK) == 0 && n < (int64_t(1) << 24)) {
      RowsX6V<T, true> pl{E + r0 * EGK, EGK, rows, K};
      ColsX6T<T, true> ql{U + k0 * n + c0, n, cols, K};
      tile_gemm_x6(acc, pl, ql, K, ldsb);
    } else {
      RowsX6V<T> pl{E + r0 * EGK, EGK, rows, K};
      ColsX6T<T> ql{U + k0 * n + c0, n, cols, K};
      tile_gemm_x6<T, 1>(acc, pl, ql, K, ldsb);
    }
  } else {
    RowsF32T<T> pl{E + r0 * EGK, EGK, rows, K, 1.f};
    ColsF32TT<T> ql{U + k0 * n + c0, n, cols, K};
    tile_gemm_pipelined(acc, pl, ql, K, lds);
  }
  if (!done) {
    if (hist && threadIdx.x < T) lrd[threadIdx.x] = 1.f / ucc;
    if (hist)
      tile_sub_from(C, n, rows, cols, acc, lds, hk);
    else
      tile_sub_from(C, n, rows, cols, acc, lds);
  }
  if (hist) {
    __syncthreads();
    for (int b = threadIdx.x; b < kSelBins; b += 256) {
      const unsigned v = lhist[b];
      if (v) atomicAdd(&hist0[b], v);
    }
  }
}

// W[:, c_begin:c_end] -= E[:, 0:K] * U[k0:k0+K, c_begin:c_end] (per row
// segment, with its U) with the tile that fills the GPU: 128 x 128 when that
// grid covers a full round of workgroups (two per CU), else 64 x 64 (four
// times the workgroups).
sg_status launch_lazy(float* W, const float* E, const Segs& segs, int64_t n, int64_t k0, int K,
                      int64_t c_begin, int64_t c_end, bool vec, hipStream_t st, unsigned* hist0 = nullptr,
                      int hist_w = 0) {
  int64_t t128 = 0, max_rows = 0;
  for (int p = 0; p < segs.n; ++p) {
    const int64_t mp = segs.row0[p + 1] - segs.row0[p];
    t128 += ceil_div(c_end - c_begin, 128) * ceil_div(mp, 128);
    max_rows = std::max<int64_t>(max_rows, mp);
  }
  if (t128 >= 2 * kNumCU) {
    const dim3 grid((unsigned)ceil_div(c_end - c_begin, 128), (unsigned)ceil_div(max_rows, 128),
                    (unsigned)segs.n);
    if (vec)
      hipLaunchKernelGGL((lazy_kernel<true, 128>), grid, dim3(256), 0, st, W, E, segs, n, k0, K, c_begin, c_end,
                         hist0, hist_w);
    else
      hipLaunchKernelGGL((lazy_kernel<false, 128>), grid, dim3(256), 0, st, W, E, segs, n, k0, K, c_begin,
                         c_end, hist0, hist_w);
  } else {
    const dim3 grid((unsigned)ceil_div(c_end - c_begin, 64), (unsigned)ceil_div(max_rows, 64),
                    (unsigned)segs.n);
    if (vec && K <= SB)
      hipLaunchKernelGGL((lazy_kernel<true, 64, true>), grid, dim3(256), 0, st, W, E, segs, n, k0, K, c_begin,
                         c_end, hist0, hist_w);
    else if (vec)
      hipLaunchKernelGGL((lazy_kernel<true, 64>), grid, dim3(256), 0, st, W, E, segs, n, k0, K, c_begin, c_end,
                         hist0, hist_w);
    else
      hipLaunchKernelGGL((lazy_kernel<false, 64>), grid, dim3(256), 0, st, W, E, segs, n, k0, K, c_begin,
                         c_end, hist0, hist_w);
  }
  return check_launch("prune lazy");
}

}  // namespace

// The 16-byte row loader of E applies when E's rows are 16-byte aligned and
// the K extent is a multiple of 4 (U is read by the 4-byte transposed loader).
bool lazy_vec(const float* E, int K) {
  return (reinterpret_cast<uintptr_t>(E) % 16) == 0 && (K % 4) == 0;
}

// Scratch of sg_prune_layer_noalloc: the prune workspace as a device array
// of the library's own, for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy (at its own address) until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// returns on that device (the array's name is a host-side stand-in there).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kScratchDevs = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevs];  // device address of `scratch`, per device
}  // namespace

sg_status noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return set_error(SG_ERR_HIP, "no current HIP device");
  if (dev >= kScratchDevs) return set_error(SG_ERR_UNSUPPORTED, "device index %d too large", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(SG_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SG_OK;
}

size_t prune_ws_bytes(int64_t m, int64_t n, int blocksize) {
  (void)n;
  (void)blocksize;
  return round_up(sizeof(SelState) * SG_MAX_SEGMENTS, 256) + round_up((size_t)m * EGK * sizeof(float), 256) +
         round_up((size_t)m * SB * sizeof(unsigned long long), 256);
}

sg_status launch_prune(const PruneArgs& a, void* ws, hipStream_t st) {
  SelState* sel = static_cast<SelState*>(ws);
  float* Err = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        round_up(sizeof(SelState) * SG_MAX_SEGMENTS, 256));
  const int64_t m = a.m, n = a.n;
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(
      reinterpret_cast<char*>(Err) + round_up((size_t)m * EGK * sizeof(float), 256));

  if (!(a.w_dtype == SG_F32 && static_cast<const void*>(a.W_out) == a.W)) {
    const size_t el = a.w_dtype == SG_BF16 ? 2 : 4;
    const int vec = (reinterpret_cast<uintptr_t>(a.W) % 16) == 0 && ((a.ldw * (int64_t)el) % 16) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.W_out) % 16) == 0 && (n % 4) == 0;
    const dim3 grid((unsigned)ceil_div(n, 2048), (unsigned)std::min<int64_t>(m, 8192));
    hipLaunchKernelGGL(convert_kernel, grid, dim3(256), 0, st, a.W_out, a.W, a.w_dtype, m, n, a.ldw, vec);
    if (sg_status e = check_launch("prune convert")) return e;
  }
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(select_pass_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(SelLds)) != hipSuccess)
    return set_error(SG_ERR_HIP, "hipFuncSetAttribute(select_pass_kernel) failed");
  const bool quant = a.bits > 0;
  const bool joint = a.vec == 16;
  const float qlevels = quant ? (float)((1 << a.bits) - 1) : 0.f;
  if (quant) {
    // grid from the original weights (W_out holds their fp32 copy)
    hipLaunchKernelGGL(qgrid_kernel, dim3((unsigned)m), dim3(256), 0, st, a.W_out, n, qlevels, a.qscale,
                       a.qzero);
    if (sg_status e = check_launch("quantization grid")) return e;
  }

  const int mode = a.mask_in ? MODE_FORCED
                             : (a.kind == SG_NM ? MODE_NM : (a.kind == SG_UNSTRUCTURED_ROW ? MODE_ROW : MODE_THRESH));
  const int B = a.blocksize;
  // segments: block-global selection runs per stacked matrix, and matrices
  // with factors of their own need their own segment; otherwise (one shared
  // factor, a mode that decides row by row) the rows form one segment
  const bool own = mode == MODE_THRESH || a.seg_u;
  Segs segs = {};
  segs.n = own ? a.nseg : 1;
  int64_t max_rows = 0;
  for (int p = 0; p < segs.n; ++p) {
    segs.row0[p] = own ? a.seg_rows[p] : 0;
    segs.row0[p + 1] = own ? a.seg_rows[p + 1] : m;
    segs.U[p] = a.seg_u ? a.Useg[p] : a.U;
    max_rows = std::max<int64_t>(max_rows, segs.row0[p + 1] - segs.row0[p]);
  }
  // Rows per lane of the column sweep: two (32 rows a workgroup) when those
  // workgroups still take one CU each, which halves each SIMD's column-step
  // work; else four (64 rows a workgroup).
  int rpl = 4;
  {
    int64_t wgs = 0;
    for (int p = 0; p < segs.n; ++p) wgs += ceil_div(segs.row0[p + 1] - segs.row0[p], 32);
    if (wgs <= kNumCU) rpl = 2;
  }
  for (int p = 0; p < segs.n; ++p)
    segs.wg0[p + 1] = segs.wg0[p] + (int)ceil_div(segs.row0[p + 1] - segs.row0[p], 16 * rpl);
  if (mode == MODE_THRESH) {
    hipLaunchKernelGGL(sel_clear_kernel, dim3((unsigned)segs.n), dim3(256), 0, st, sel);
    if (sg_status e = check_launch("select clear")) return e;
  }
  // select: enough workgroups that every thread holds at most SEL_KPT keys
  const dim3 sel_grid((unsigned)std::max<int64_t>(1, ceil_div(max_rows, (int64_t)2 * SEL_KPT)),
                      (unsigned)segs.n);
  const dim3 sw_grid((unsigned)segs.wg0[segs.n]);
  // lazy-update groups: GK columns (a multiple of the block width, at most EGK)
  const int64_t GK = (EGK / B) * B;
  int parity = 0;
  // the first radix pass of a block is taken in the epilogue of the lazy
  // update that produces its final values when there is one matrix
  bool pass0_done = false;
  for (int64_t i1 = 0; i1 < n; i1 += B, parity ^= 1) {
    const int w = (int)std::min<int64_t>(B, n - i1);
    const int64_t g0 = (i1 / GK) * GK;
    const int64_t g_end = std::min<int64_t>(n, g0 + GK);
    float* Eb = Err + (i1 - g0);  // this block's columns of the group's error buffer
    if (mode == MODE_THRESH) {
      bool any = false;
      for (int p = 0; p < segs.n; ++p) {
        const int64_t mp = segs.row0[p + 1] - segs.row0[p];
        const long long k = (long long)floor(a.sparsity * (double)mp * (double)w);
        segs.k[p] = k;
        segs.fixed[p] = k <= 0 ? 2 : (k >= (long long)mp * w ? 3 : 0);
        any = any || segs.fixed[p] == 0;
      }
      if (any) {
        for (int pass = pass0_done ? 1 : 0; pass < 2; ++pass) {
          hipLaunchKernelGGL(select_pass_kernel, sel_grid, dim3(256), sizeof(SelLds), st, sel, parity,
                             cand, static_cast<const float*>(a.W_out), segs, n, i1, w, pass);
          if (sg_status e = check_launch("select pass")) return e;
        }
      }
    }
    SweepArgs sa;
    sa.W = a.W_out;
    sa.mask_out = a.mask_out;
    sa.Err = Eb;
    sa.mask_in = a.mask_in;
    sa.st = sel;
    sa.cand = cand;
    sa.parity = parity;
    sa.segs = segs;
    sa.n = n;
    sa.i1 = i1;
    sa.w = w;
    sa.nkeep = a.n_keep;
    sa.mgroup = a.m_group;
    sa.codes_out = a.codes_out;
    sa.qscale = a.qscale;
    sa.qzero = a.qzero;
    sa.qlevels = qlevels;
    sa.mode = mode;
    sa.mgs = 0;
    sa.rpl = rpl;
    sa.grid = sw_grid;
    sa.stream = st;
    if (mode == MODE_NM && a.m_group <= 16) sa.mgs = a.m_group;
    if (mode == MODE_ROW) {
      // one group per row spanning the block: keep w - floor(p * w)
      sa.nkeep = w - (int)floor(a.sparsity * (double)w);
      sa.mgroup = w;
    }
    if (sg_status e = quant ? launch_sweep_quant(sa) : (joint ? launch_sweep_joint(sa) : launch_sweep_plain(sa)))
      return e;
    const int64_t i2 = i1 + w;
    // next block: histogram its keys' top digit in the lazy update's epilogue?
    unsigned* hist0 = nullptr;
    int hist_w = 0;
    if (mode == MODE_THRESH && segs.n == 1 && i2 < n) {
      const int w2 = (int)std::min<int64_t>(B, n - i2);
      const long long k2 = (long long)floor(a.sparsity * (double)m * (double)w2);
      if (k2 > 0 && k2 < (long long)m * w2) {
        hist0 = sel[0].set[parity ^ 1].hist0;
        hist_w = w2;
      }
    }
    pass0_done = hist0 != nullptr;
    if (i2 < g_end) {
      // rest of the group, K = block width
      if (sg_status e =
              launch_lazy(a.W_out, Eb, segs, n, i1, w, i2, g_end, lazy_vec(Eb, w), st, hist0, hist_w))
        return e;
    } else if (g_end < n) {
      // last block of the group: every column beyond it, K = group width
      if (sg_status e = launch_lazy(a.W_out, Err, segs, n, g0, (int)(g_end - g0), g_end, n,
                                    lazy_vec(Err, (int)(g_end - g0)), st, hist0, hist_w))
        return e;
    } else {
      pass0_done = false;
    }
  }
  return SG_OK;
}

}  // namespace sg
