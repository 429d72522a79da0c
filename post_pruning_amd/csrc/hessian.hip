// Hessian accumulation H += Xc^T Xc on gfx950.
//
// "SparseGPT ... Pruned in One-Shot" review (devpress), section 7: the layer's
// second-order information is H = X X^T of its calibration inputs.  X arrives
// token-major, Xc[t, c], so H[i][j] = sum_t Xc[t][i] Xc[t][j]: a symmetric
// rank-T update whose reduction axis (tokens) is the strided one.
//
// bf16 path: 256x256 output tiles of the lower triangle only (the symmetric
// result is mirrored on store), 8 waves per workgroup, each wave a 128x64
// sub-tile of v_mfma_f32_16x16x32_bf16 (two waves per SIMD).  X tiles are staged through LDS in
// column-major form (each LDS row = one channel, 64 consecutive tokens) by an
// in-register 8x8 transpose, so every MFMA operand is one 16-byte LDS read.
// When there are too few tiles to fill the 256 CUs the tokens are split; every
// split writes its partial tile to the workspace and the last split to finish
// sums all partials in split order (bitwise reproducible), then adds into H.
#include "sg_internal.h"

#include <math.h>

#include <algorithm>

namespace sg {
namespace {

constexpr int HT = kHessTile;          // 256
constexpr int HBK = 64;                // tokens per LDS stage
constexpr int HROWB = HBK * 2 + 16;    // LDS bytes per channel row (padded)
constexpr int HTHREADS = 512;
constexpr int kMinTokPerSplit = 4096;

__device__ inline void tri_decode(int64_t ti, int& I, int& J) {
  int64_t r = (int64_t)((sqrt(8.0 * (double)ti + 1.0) - 1.0) * 0.5);
  while ((r + 1) * (r + 2) / 2 <= ti) ++r;
  while (r * (r + 1) / 2 > ti) --r;
  I = (int)r;
  J = (int)(ti - r * (r + 1) / 2);
}

__global__ void zero_u32_kernel(unsigned* p, int64_t cnt) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < cnt) p[i] = 0u;
}

__device__ inline float agent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool RAGGED>
__global__ __launch_bounds__(HTHREADS) void hess_bf16_kernel(
    float* __restrict__ H, int n, const uint16_t* __restrict__ X, int64_t T,
    int64_t ldx, int64_t tiles, int splits, int64_t tps,
    float* __restrict__ part, unsigned* __restrict__ counters) {
  // Two LDS stages (double buffer), each holding the I-block and the J-block.
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2 * HT * HROWB];
  __shared__ int s_last;

  // Work items are split-major (item = split * tiles + tile) and taken in
  // launch order: the workgroups resident at any time all stream the same
  // token range, spread over all 8 XCDs, so each X slice is fetched from HBM
  // once into the shared Infinity Cache.  (Grouping tiles per XCD to favour
  // the per-XCD L2 measured slower.)
  const int64_t item = blockIdx.x;
  const int split = (int)(item / tiles);
  const int64_t ti = item - (int64_t)split * tiles;
  int I, J;
  tri_decode(ti, I, J);
  const bool diag = (I == J);
  const int i0 = I * HT, j0 = J * HT;
  const int64_t t_begin = (int64_t)split * tps;
  const int64_t t_end = min(T, t_begin + tps);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wi = wave >> 2;  // 128-row half of the tile
  const int wj = wave & 3;   // 64-column quarter

  // Loader role: threads 0..255 stage the I-block, 256..511 the J-block (only
  // for off-diagonal tiles), one 8 tokens x 8 channels block each per stage.
  const int op = tid >> 8;
  const int tb = tid & 7;          // 8-token group inside the stage
  const int cb = (tid & 255) >> 3; // 8-channel group inside the tile
  const bool loader = !(diag && op == 1);

  floatx4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  u32x4 r[8];

  // All loads of a stage are issued back to back from clamped, always
  // in-bounds addresses (rows past the token range re-read the last row,
  // channel groups past n re-read the last group); out-of-range data is
  // zeroed only when the stage is written to LDS, so no load waits on another.
  // Per stage one uniform base pointer (row t0) and 32-bit per-lane byte
  // offsets: SGPR-base addressing, no 64-bit address registers.
  // RAGGED (n not a multiple of 8) takes a per-element path instead.
  auto gload = [&](int64_t t0) {
    if (!loader) return;
    const char* base = reinterpret_cast<const char*>(X + t0 * ldx);
    const bool partial = t0 + HBK > t_end;
    const int last = (int)(t_end - 1 - t0);
    const int colbase = (op == 0 ? i0 : j0) + cb * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int tr = tb * 8 + i;
      if (partial) tr = tr < last ? tr : last;
      if constexpr (!RAGGED) {
        const int colc = colbase < n ? colbase : n - 8;
        const uint32_t off = (uint32_t)tr * (uint32_t)(ldx * 2) + (uint32_t)colc * 2u;
        r[i] = *reinterpret_cast<const u32x4*>(base + off);
      } else {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        const uint16_t* src =
            reinterpret_cast<const uint16_t*>(base + (uint32_t)tr * (uint32_t)(ldx * 2));
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (colbase + e < n) v[e >> 1] |= (uint32_t)src[colbase + e] << (16 * (e & 1));
        r[i] = v;
      }
    }
  };

  // Transpose the 8x8 block in registers and store it channel-major.
  auto lstore = [&](int64_t t0, unsigned char* buf) {
    if (!loader) return;
    unsigned char* dst = buf + op * HT * HROWB;
    const bool colok = ((op == 0 ? i0 : j0) + cb * 8) < n;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = colok && (t0 + tb * 8 + i) < t_end;
      if (!ok) r[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 lo, hi;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const uint32_t a0 = r[2 * qq][d], a1 = r[2 * qq + 1][d];
        lo[qq] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
        hi[qq] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
      }
      *reinterpret_cast<u32x4*>(dst + (cb * 8 + 2 * d) * HROWB + tb * 16) = lo;
      *reinterpret_cast<u32x4*>(dst + (cb * 8 + 2 * d + 1) * HROWB + tb * 16) = hi;
    }
  };

  auto compute = [&](const unsigned char* buf, int ks) {
    const unsigned char* la = buf;
    const unsigned char* lb = diag ? buf : buf + HT * HROWB;
    const int koff = ks * 64 + (lane >> 4) * 16;
    bf16x8 fb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      fb[c] = *reinterpret_cast<const bf16x8*>(lb + (wj * 64 + c * 16 + (lane & 15)) * HROWB + koff);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const bf16x8 fa =
          *reinterpret_cast<const bf16x8*>(la + (wi * 128 + a * 16 + (lane & 15)) * HROWB + koff);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c], acc[a][c], 0, 0, 0);
    }
  };

  // Software pipeline: stage s is computed from LDS buffer s%2 while stage
  // s+1 (already in registers) is written to the other buffer half-way
  // through, and stage s+2 is then fetched into registers.  One barrier per
  // stage.
  const int64_t ntok = t_end > t_begin ? t_end - t_begin : 0;
  const int64_t nsteps = ceil_div(ntok, HBK);
  if (nsteps > 0) {
    gload(t_begin);
    lstore(t_begin, lds[0]);
    if (nsteps > 1) gload(t_begin + HBK);
    __syncthreads();
  }
  for (int64_t step = 0; step < nsteps; ++step) {
    unsigned char* cur = lds[step & 1];
    unsigned char* nxt = lds[(step + 1) & 1];
    compute(cur, 0);
    if (step + 1 < nsteps) {
      lstore(t_begin + (step + 1) * HBK, nxt);
      if (step + 2 < nsteps) gload(t_begin + (step + 2) * HBK);
    }
    compute(cur, 1);
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  if (splits > 1) {
    // Partial tile layout: per (wave, a, c) slot, 64 lanes x float4.
    floatx4* mine = reinterpret_cast<floatx4*>(part + (size_t)item * (HT * HT));
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) mine[(wave * 32 + a * 4 + c) * 64 + lane] = acc[a][c];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned old = atomicAdd(&counters[ti], 1u);
      s_last = (old == (unsigned)(splits - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // Sum the partials of every split of this tile in split order (the own
    // partial is re-read too, so the order and the result do not depend on
    // which split finished last).
    for (int sp = 0; sp < splits; ++sp) {
      const floatx4* other =
          reinterpret_cast<const floatx4*>(part + ((size_t)sp * tiles + ti) * (HT * HT));
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const floatx4 pv = other[(wave * 32 + a * 4 + c) * 64 + lane];
          acc[a][c] = (sp == 0) ? pv : acc[a][c] + pv;
        }
    }
    if (tid == 0) counters[ti] = 0u;
  }

#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i0 + wi * 128 + a * 16 + (lane >> 4) * 4 + v;
        const int col = j0 + wj * 64 + c * 16 + (lane & 15);
        if (row >= n || col >= n) continue;
        if (diag && row < col) continue;
        const size_t lo = (size_t)row * n + col;
        const float val = H[lo] + acc[a][c][v];
        H[lo] = val;
        if (row != col) H[(size_t)col * n + row] = val;
      }
}

// fp32 inputs: plain LDS-tiled VALU kernel (64x64 lower tiles, 4x4 outputs
// per thread).  Each 32-token stage is summed separately before it is added
// to the running total.
constexpr int FT = 64;
constexpr int FBK = 32;

__global__ __launch_bounds__(256) void hess_f32_kernel(float* __restrict__ H, int n,
                                                       const float* __restrict__ X,
                                                       int64_t T, int64_t ldx) {
  __shared__ float As[FBK][FT + 4];
  __shared__ float Bs[FBK][FT + 4];
  int I, J;
  tri_decode(blockIdx.x, I, J);
  const int i0 = I * FT, j0 = J * FT;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t t0 = 0; t0 < T; t0 += FBK) {
    for (int e = threadIdx.x; e < FBK * FT; e += 256) {
      const int tt = e / FT, c = e % FT;
      const int64_t t = t0 + tt;
      As[tt][c] = (t < T && i0 + c < n) ? X[t * ldx + i0 + c] : 0.f;
      Bs[tt][c] = (t < T && j0 + c < n) ? X[t * ldx + j0 + c] : 0.f;
    }
    __syncthreads();
    float stage[4][4] = {};
    for (int k = 0; k < FBK; ++k) {
      float a[4], bb[4];
      for (int u = 0; u < 4; ++u) a[u] = As[k][ty * 4 + u];
      for (int u = 0; u < 4; ++u) bb[u] = Bs[k][tx * 4 + u];
      for (int u = 0; u < 4; ++u)
        for (int w = 0; w < 4; ++w) stage[u][w] = fmaf(a[u], bb[w], stage[u][w]);
    }
    for (int u = 0; u < 4; ++u)
      for (int w = 0; w < 4; ++w) acc[u][w] += stage[u][w];
    __syncthreads();
  }
  for (int u = 0; u < 4; ++u)
    for (int w = 0; w < 4; ++w) {
      const int row = i0 + ty * 4 + u, col = j0 + tx * 4 + w;
      if (row >= n || col >= n) continue;
      if (I == J && row < col) continue;
      const size_t lo = (size_t)row * n + col;
      const float val = H[lo] + acc[u][w];
      H[lo] = val;
      if (row != col) H[(size_t)col * n + row] = val;
    }
}

}  // namespace

HessPlan hessian_plan(int64_t n, int64_t T, size_t ws_avail, bool limit_by_ws) {
  HessPlan p;
  const int64_t nt = ceil_div(n, HT);
  p.tiles = nt * (nt + 1) / 2;
  const size_t tile_bytes = (size_t)HT * HT * sizeof(float);
  const size_t cnt_bytes = round_up(p.tiles * sizeof(unsigned), 256);
  int max_s = (int)std::max<int64_t>(1, std::min<int64_t>(64, T / kMinTokPerSplit));
  if (limit_by_ws) {
    if (ws_avail <= cnt_bytes) {
      max_s = 1;
    } else {
      const int64_t fit = (int64_t)((ws_avail - cnt_bytes) / (tile_bytes * (size_t)p.tiles));
      max_s = (int)std::max<int64_t>(1, std::min<int64_t>(max_s, fit));
    }
  }
  // Pick the split count that best fills whole waves of workgroups (one
  // 512-thread workgroup per CU), with a small penalty per split for the
  // partial-tile traffic.
  double best = 1e300;
  int best_s = 1;
  for (int s = 1; s <= max_s; ++s) {
    const double rounds = (double)ceil_div(p.tiles * s, kNumCU);
    const double score = rounds / s * (1.0 + 0.005 * s);
    if (score < best * 0.999) {
      best = score;
      best_s = s;
    }
  }
  p.splits = best_s;
  p.tok_per_split = round_up(ceil_div(T, best_s), HBK);
  // Recompute the split count actually needed with the rounded split size.
  p.splits = (int)std::max<int64_t>(1, ceil_div(T, p.tok_per_split));
  p.ws_bytes = p.splits > 1 ? cnt_bytes + tile_bytes * (size_t)p.tiles * p.splits : 0;
  return p;
}

sg_status launch_hessian_bf16(float* H, int64_t n, const uint16_t* X, int64_t T,
                              int64_t ldx, const HessPlan& plan, void* ws,
                              hipStream_t st) {
  unsigned* counters = nullptr;
  float* part = nullptr;
  if (plan.splits > 1) {
    counters = reinterpret_cast<unsigned*>(ws);
    part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                    round_up(plan.tiles * sizeof(unsigned), 256));
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)ceil_div(plan.tiles, 256)), dim3(256),
                       0, st, counters, plan.tiles);
    if (sg_status e = check_launch("hessian counters")) return e;
  }
  const int64_t grid = plan.tiles * plan.splits;
  if (n % 8 == 0)
    hipLaunchKernelGGL(hess_bf16_kernel<false>, dim3((unsigned)grid), dim3(HTHREADS), 0, st, H,
                       (int)n, X, T, ldx, plan.tiles, plan.splits, plan.tok_per_split, part, counters);
  else
    hipLaunchKernelGGL(hess_bf16_kernel<true>, dim3((unsigned)grid), dim3(HTHREADS), 0, st, H,
                       (int)n, X, T, ldx, plan.tiles, plan.splits, plan.tok_per_split, part, counters);
  return check_launch("hessian bf16");
}

sg_status launch_hessian_f32(float* H, int64_t n, const float* X, int64_t T, int64_t ldx,
                             hipStream_t st) {
  const int64_t nt = ceil_div(n, FT);
  const int64_t tiles = nt * (nt + 1) / 2;
  hipLaunchKernelGGL(hess_f32_kernel, dim3((unsigned)tiles), dim3(256), 0, st, H, (int)n, X, T,
                     ldx);
  return check_launch("hessian f32");
}

}  // namespace sg
