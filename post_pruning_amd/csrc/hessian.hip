// Hessian accumulation H += Xc^T Xc on gfx950.
//
// "SparseGPT ... Pruned in One-Shot" review (devpress), section 7: the layer's
// second-order information is H = X X^T of its calibration inputs.  X arrives
// token-major, Xc[t, c], so H[i][j] = sum_t Xc[t][i] Xc[t][j]: a symmetric
// rank-T update whose reduction axis (tokens) is the strided one.
//
// bf16 path: 256x256 output tiles of the lower triangle only (the symmetric
// result is mirrored on store), 8 waves per workgroup, each wave a 128x64
// sub-tile of v_mfma_f32_16x16x32_bf16 (two waves per SIMD).  Two kernels
// stage X through LDS:
//   * hess_bf16_dma_kernel (n % 8 == 0, the main path): token rows are copied
//     as they lie in X straight from global memory into LDS by the LDS-DMA
//     loads, and the operands are gathered by the transposing LDS read;
//   * hess_bf16_kernel (any n): tiles are transposed in registers (8x8) and
//     stored channel-major (each LDS row = one channel, 64 consecutive
//     tokens), so every MFMA operand is one 16-byte LDS read.
// When there are too few tiles to fill the 256 CUs the tokens are split; every
// split writes its partial tile to the workspace and the last split to finish
// sums all partials in split order (bitwise reproducible), then adds into H.
//
// Tile order: the hardware deals workgroups round-robin over the 8 XCDs, each
// with its own L2.  Tiles are enumerated in g x g groups of panels (panel =
// 256 channels), and XCD x takes a contiguous eighth of that order, split-major:
// the workgroups resident on one XCD then work on a compact set of tiles that
// share few panels, over the same token range, so most X re-reads hit its L2;
// the XCDs run the same token range at the same time, which the shared
// Infinity Cache serves once.
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

// k-th tile of the grouped order: panel rows in blocks of g; inside a block
// row BI, the off-diagonal g x g groups (BJ < BI) row-major, then the
// diagonal group's lower triangle.
__device__ inline void grouped_decode(int64_t k, int nt, int g, int& I, int& J) {
  int64_t base = 0;
  for (int BI = 0;; ++BI) {
    const int r0 = BI * g;
    const int gi = min(g, nt - r0);
    const int64_t off = (int64_t)BI * gi * g;
    const int64_t row = off + (int64_t)gi * (gi + 1) / 2;
    if (k < base + row || r0 + gi >= nt) {
      const int64_t rem = k - base;
      if (rem < off) {
        const int64_t per = (int64_t)gi * g;
        const int BJ = (int)(rem / per);
        const int r2 = (int)(rem - BJ * per);
        I = r0 + r2 / g;
        J = BJ * g + r2 % g;
      } else {
        int a, b;
        tri_decode(rem - off, a, b);
        I = r0 + a;
        J = r0 + b;
      }
      return;
    }
    base += row;
  }
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
    int64_t ldx, int64_t tiles, int splits, int64_t tps, int group,
    float* __restrict__ part, unsigned* __restrict__ counters) {
  // Two LDS stages (double buffer), each holding the I-block and the J-block.
  // Separate arrays, so the compiler can tell the stage being written from the
  // stage being read and interleave the two.
  __shared__ __attribute__((aligned(16))) unsigned char lds0[2 * HT * HROWB];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[2 * HT * HROWB];
  __shared__ int s_last;

  // XCD share: tiles [k0, k1) of the grouped order, times all splits,
  // split-major.  Shares differ by at most one tile; the few workgroups past
  // a short share exit at once.
  const int xcd = blockIdx.x & 7;
  const int64_t jx = blockIdx.x >> 3;
  const int64_t k0 = tiles * xcd / 8, k1 = tiles * (xcd + 1) / 8;
  const int64_t cnt = k1 - k0;
  if (jx >= cnt * splits) return;
  const int split = (int)(jx / cnt);
  const int64_t ti = k0 + (jx - (int64_t)split * cnt);
  const int64_t item = (int64_t)split * tiles + ti;
  int I, J;
  grouped_decode(ti, (int)ceil_div((int64_t)n, HT), group, I, J);
  const bool diag = (I == J);
  const int i0 = I * HT, j0 = J * HT;
  const int64_t t_begin = (int64_t)split * tps;
  const int64_t t_end = min(T, t_begin + tps);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wi = wave >> 2;  // 128-row half of the tile
  const int wj = wave & 3;   // 64-column quarter

  // Loader role: threads 0..255 stage the I-block, 256..511 the J-block (a
  // second copy of the I-block on diagonal tiles, which keeps every step
  // free of branches), one 8 tokens x 8 channels block each per stage.
  const int op = tid >> 8;
  const int tb = tid & 7;          // 8-token group inside the stage
  const int cb = (tid & 255) >> 3; // 8-channel group inside the tile
  const int colbase = (op == 0 ? i0 : j0) + cb * 8;
  const bool colok = colbase < n;

  floatx4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  u32x4 r[8];

  // Generic stage load (first and last stages): clamped, always in-bounds
  // addresses (rows past the token range re-read the last row, channel groups
  // past n re-read the last group); out-of-range data is zeroed when the stage
  // is written to LDS.  RAGGED (n not a multiple of 8) loads per element.
  auto gload = [&](int64_t t0) {
    const char* base = reinterpret_cast<const char*>(X + t0 * ldx);
    const int last = (int)min<int64_t>(HBK - 1, t_end - 1 - t0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int tr = tb * 8 + i;
      tr = tr < last ? tr : last;
      if constexpr (!RAGGED) {
        const int colc = colok ? colbase : n - 8;
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

  // Transpose the 8x8 block in registers and store it channel-major: one
  // 16-byte LDS write per pair of channels (d selects channels 2d, 2d+1).
  auto lstore_pair = [&](unsigned char* dst, int d) {
    u32x4 lo, hi;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint32_t a0 = r[2 * qq][d], a1 = r[2 * qq + 1][d];
      lo[qq] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
      hi[qq] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    }
    *reinterpret_cast<u32x4*>(dst + (cb * 8 + 2 * d) * HROWB + tb * 16) = lo;
    *reinterpret_cast<u32x4*>(dst + (cb * 8 + 2 * d + 1) * HROWB + tb * 16) = hi;
  };

  auto lstore = [&](int64_t t0, unsigned char* buf) {
    unsigned char* dst = buf + op * HT * HROWB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = colok && (t0 + tb * 8 + i) < t_end;
      if (!ok) r[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) lstore_pair(dst, d);
  };

  // MFMA operands: lane l reads 16 bytes (8 tokens) of channel row l%16 at
  // token offset 8*(l/16) inside the 32-token half ks of the stage.
  const int koff = (lane >> 4) * 16;
  const int arow = (wi * 128 + (lane & 15)) * HROWB + koff;
  const int brow = HT * HROWB + (wj * 64 + (lane & 15)) * HROWB + koff;

  auto compute = [&](const unsigned char* buf, int ks) {
    bf16x8 fb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      fb[c] = *reinterpret_cast<const bf16x8*>(buf + brow + c * 16 * HROWB + ks * 64);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const bf16x8 fa = *reinterpret_cast<const bf16x8*>(buf + arow + a * 16 * HROWB + ks * 64);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c], acc[a][c], 0, 0, 0);
    }
  };

  // Steady-state step (all tokens of the stages involved valid): compute
  // stage s from `cur`, write stage s+1 (in registers) to `nxt`, fetch stage
  // s+2 into registers.  No branches and no bounds selects; the scheduling
  // groups interleave the LDS writes, the transposes and the global loads
  // with the 64 MFMAs of the step so that they issue while the matrix core
  // is busy.
  const uint32_t loff =
      (uint32_t)(tb * 8) * (uint32_t)(ldx * 2) + (uint32_t)(colok ? colbase : n - 8) * 2u;
  auto fast_step = [&](const unsigned char* cur, unsigned char* nxt, int64_t t_load) {
    // half 1: 32 MFMA (k = 0..31 of the stage) with their 12 operand reads,
    // interleaved with the 32 transposes and 8 LDS writes of the next stage
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, 0);
    unsigned char* dst = nxt + op * HT * HROWB;
#pragma unroll
    for (int d = 0; d < 4; ++d) lstore_pair(dst, d);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (g < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // half 2: 32 MFMA (k = 32..63) with their operand reads, interleaved with
    // the 8 global loads of stage s+2 (into the registers just written out)
    const char* base = reinterpret_cast<const char*>(X + t_load * ldx);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = *reinterpret_cast<const u32x4*>(base + (size_t)i * (size_t)(ldx * 2) + loff);
    compute(cur, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      if (g < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };

  // Software pipeline: stage s is computed from LDS buffer s%2 while stage
  // s+1 (already in registers) is written to the other buffer, and stage s+2
  // is fetched into registers.  One barrier per stage.
  const int64_t ntok = t_end > t_begin ? t_end - t_begin : 0;
  const int64_t nsteps = ceil_div(ntok, HBK);
  const int64_t nfull = ntok / HBK;
  if (nsteps > 0) {
    gload(t_begin);
    lstore(t_begin, lds0);
    if (nsteps > 1) gload(t_begin + HBK);
    __syncthreads();
  }
  int64_t step = 0;
  if constexpr (!RAGGED) {
    // pairs of steady-state steps: step s + 2 (and s + 3) must be full stages
    for (; step + 3 < nfull; step += 2) {
      fast_step(lds0, lds1, t_begin + (step + 2) * HBK);
      fast_step(lds1, lds0, t_begin + (step + 3) * HBK);
    }
  }
  for (; step < nsteps; ++step) {
    unsigned char* cur = (step & 1) ? lds1 : lds0;
    unsigned char* nxt = (step & 1) ? lds0 : lds1;
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

// bf16 path for n % 8 == 0: the same tiles and wave layout, with the X
// stages copied straight from global memory into LDS by the LDS-DMA loads
// (no register staging, no transposes in VALU).  A stage is 32 tokens; in
// LDS each token is one 1040-byte row holding the tile's I-panel (256
// channels) and J-panel (256 channels) as they lie in X, plus 16 bytes of
// padding so that consecutive tokens start 16 bytes apart in the LDS banks.
// MFMA operands (8 consecutive tokens of one channel per lane) are read with
// the transposing LDS read, which gathers 4 tokens x 4 channels across 16
// lanes.  Four stages rotate, three in flight while the fourth is multiplied.
constexpr int DK = 32;                       // tokens per stage
constexpr int DROW = 2 * HT * 2 + 16;        // LDS bytes per token row
constexpr int DSTAGE = DK * DROW;            // 33280 bytes per stage

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// s_waitcnt immediates that wait for the vector-memory counter only.
constexpr unsigned kWaitVm0 = 0x0F70u;
constexpr unsigned kWaitVm4 = 0x0F74u;
constexpr unsigned kWaitVm8 = 0x0F78u;

// One LDS-DMA copy: lane l moves 16 bytes from gbase + voff (its own offset)
// to LDS byte address lds_addr + 16 * l.  Issued from inline assembly so that
// the compiler does not add waits of its own for the copies (it cannot tell
// which stage a later LDS read touches at the head of the software-pipelined
// loop and would wait for every copy in flight); all ordering of the copies
// is explicit (s_waitcnt vmcnt before the barrier that publishes a stage).
// The instruction has no register results; M0 is used by nothing else here.
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory", "m0");
}

// Workgroup barrier without a memory fence: a fence would also wait for the
// stages still in flight.  LDS visibility is ordered by hand (each wave waits
// for its own copies of a stage before the barrier that publishes it); the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ inline void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(HTHREADS) void hess_bf16_dma_kernel(
    float* __restrict__ H, int n, const uint16_t* __restrict__ X, int64_t T,
    int64_t ldx, int64_t tiles, int splits, int64_t tps, int group,
    float* __restrict__ part, unsigned* __restrict__ counters) {
  // One array per stage.
  __shared__ __attribute__((aligned(16))) unsigned char st0[DSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[DSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[DSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st3[DSTAGE];
  __shared__ int s_last;

  const int xcd = blockIdx.x & 7;
  const int64_t jx = blockIdx.x >> 3;
  const int64_t k0 = tiles * xcd / 8, k1 = tiles * (xcd + 1) / 8;
  const int64_t cnt = k1 - k0;
  if (jx >= cnt * splits) return;
  const int split = (int)(jx / cnt);
  const int64_t ti = k0 + (jx - (int64_t)split * cnt);
  const int64_t item = (int64_t)split * tiles + ti;
  int I, J;
  grouped_decode(ti, (int)ceil_div((int64_t)n, HT), group, I, J);
  const bool diag = (I == J);
  const int i0 = I * HT, j0 = J * HT;
  const int64_t t_begin = (int64_t)split * tps;
  const int64_t t_end = min(T, t_begin + tps);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wi = wave >> 2;
  const int wj = wave & 3;

  floatx4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Copy role: wave w copies token rows 4w..4w+3 of every stage, one row per
  // instruction; lanes 0..31 fetch the I-panel's 32 16-byte chunks, lanes
  // 32..63 the J-panel's (on diagonal tiles a second copy of the I-panel).
  // Channel chunks past n re-read the last chunk: those channels only feed
  // outputs beyond n, which are never stored.
  int col = ((lane >> 5) ? j0 : i0) + (lane & 31) * 8;
  col = col < n ? col : n - 8;
  const uint32_t dcol = (uint32_t)col * 2u;
  auto copy_stage = [&](unsigned char* buf, int64_t s) {
    const int64_t tok0 = t_begin + s * DK + wave * 4;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)buf + (uint32_t)(wave * 4 * DROW);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t t = tok0 + j;
      t = t < t_end ? t : t_end - 1;  // rows past the end are zeroed later
      const char* row = reinterpret_cast<const char*>(X) + t * ldx * 2;
      lds_dma16(row, dcol, __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(j * DROW)));
    }
  };

  // Operand addresses: lane l of a transposing read points at token row
  // 8*(l/16) + (l%16)/4 (+4 for the second read) and channel quad l%4 of the
  // 16-channel fragment; lane i of the result then holds channel i of the
  // fragment over those 4 tokens.
  const int s16 = lane & 15;
  const int trow = 8 * (lane >> 4) + (s16 >> 2);
  const int q4 = 4 * (s16 & 3);
  const uint32_t a_off = (uint32_t)(trow * DROW + (wi * 128 + q4) * 2);
  const uint32_t b_off = (uint32_t)(trow * DROW + HT * 2 + (wj * 64 + q4) * 2);

  auto frag = [&](const unsigned char* buf, uint32_t off) {
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(buf + off));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(buf + off + 4 * DROW));
    const shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  };

  auto compute = [&](const unsigned char* buf) {
    bf16x8 fb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) fb[c] = frag(buf, b_off + c * 32);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const bf16x8 fa = frag(buf, a_off + a * 32);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[c], acc[a][c], 0, 0, 0);
    }
  };

  const int64_t ntok = t_end > t_begin ? t_end - t_begin : 0;
  const int64_t nsteps = ceil_div(ntok, DK);
  if (nsteps > 0) copy_stage(st0, 0);
  if (nsteps > 1) copy_stage(st1, 1);
  if (nsteps > 2) copy_stage(st2, 2);

  // Steady-state step s (fragments of stage s already in registers, stage s
  // complete in LDS): wait for this wave's copies of stage s+1 (stage s+2 may
  // stay in flight), barrier (stage s+1 complete; every wave is done with
  // stage s-1), start copying stage s+3 into the buffer of stage s-1,
  // multiply stage s, and read the first fragments of stage s+1, so that the
  // next step's MFMAs start right after its barrier.
  struct Frags {
    bf16x8 fb[4];
    bf16x8 fa0;
  };
  auto prefetch = [&](const unsigned char* buf, Frags& f) {
#pragma unroll
    for (int c = 0; c < 4; ++c) f.fb[c] = frag(buf, b_off + c * 32);
    f.fa0 = frag(buf, a_off);
  };
  auto step = [&](const unsigned char* cur, const unsigned char* nxt, unsigned char* refill,
                  int64_t s, Frags& f) {
    __builtin_amdgcn_s_waitcnt(kWaitVm4);
    stage_barrier();
    copy_stage(refill, s + 3);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 fa = f.fa0;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const bf16x8 fan = a < 7 ? frag(cur, a_off + (a + 1) * 32) : fa;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f.fb[c], acc[a][c], 0, 0, 0);
      fa = fan;
    }
    prefetch(nxt, f);
    // two operand reads ahead of the MFMAs; the next stage's fragments are
    // read during the last MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int64_t s = 0;
  if (nsteps > 6) {
    __builtin_amdgcn_s_waitcnt(kWaitVm4);  // stages 0 and 1
    stage_barrier();
    Frags f;
    prefetch(st0, f);
    for (; s + 6 < nsteps; s += 4) {
      step(st0, st1, st3, s, f);
      step(st1, st2, st0, s + 1, f);
      step(st2, st3, st1, s + 2, f);
      step(st3, st0, st2, s + 3, f);
    }
  }
  for (; s < nsteps; ++s) {
    const int b = (int)(s & 3);
    unsigned char* cur = b == 0 ? st0 : b == 1 ? st1 : b == 2 ? st2 : st3;
    unsigned char* refill = b == 0 ? st3 : b == 1 ? st0 : b == 2 ? st1 : st2;
    const int64_t later = nsteps - 1 - s;
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(kWaitVm4);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stage_barrier();
    const int valid = (int)min<int64_t>(DK, ntok - s * DK);
    if (valid < DK) {
      // last, partial stage: zero the token rows past the end
      for (int e = tid; e < (DK - valid) * (DROW / 16); e += HTHREADS) {
        const int row = valid + e / (DROW / 16);
        *reinterpret_cast<u32x4*>(cur + row * DROW + (e % (DROW / 16)) * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (s + 3 < nsteps) copy_stage(refill, s + 3);
    compute(cur);
  }

  // ---- epilogue (same layout as the register-staged kernel) ---------------
  if (splits > 1) {
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
    for (int sp = 0; sp < splits; ++sp) {
      const floatx4* other =
          reinterpret_cast<const floatx4*>(part + ((size_t)sp * tiles + ti) * (HT * HT));
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        floatx4 pv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) pv[c] = other[(wave * 32 + a * 4 + c) * 64 + lane];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = (sp == 0) ? pv[c] : acc[a][c] + pv[c];
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
        const int col2 = j0 + wj * 64 + c * 16 + (lane & 15);
        if (row >= n || col2 >= n) continue;
        if (diag && row < col2) continue;
        const size_t lo = (size_t)row * n + col2;
        const float val = H[lo] + acc[a][c][v];
        H[lo] = val;
        if (row != col2) H[(size_t)col2 * n + row] = val;
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
  // 512-thread workgroup per CU), with a penalty of 2% per split for the
  // partial tiles (their writes, and the serial sum in the last split).
  // Measured at n = 4096, T = 262144: 7 splits (4 rounds, 93% full) take
  // 4.50-4.60 ms, 15 splits (8 rounds, 99.6% full) 4.63-4.73 ms.
  double best = 1e300;
  int best_s = 1;
  for (int s = 1; s <= max_s; ++s) {
    const double rounds = (double)ceil_div(p.tiles * s, kNumCU);
    const double score = rounds / s * (1.0 + 0.02 * s);
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
  // Group edge: about the square root of the tiles an XCD has resident at once
  // (its 32 CUs, or its whole share when that is smaller).
  const double per_xcd = std::min<double>(32.0, (double)p.tiles * p.splits / 8.0) /
                         std::max(1, std::min(p.splits, 2));
  p.group = (int)std::max<int64_t>(1, std::min<int64_t>(nt, (int64_t)std::lround(std::sqrt(per_xcd))));
  p.grid = 8 * ceil_div(p.tiles, 8) * p.splits;
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
  const int64_t grid = plan.grid;
  if (n % 8 == 0)
    hipLaunchKernelGGL(hess_bf16_dma_kernel, dim3((unsigned)grid), dim3(HTHREADS), 0, st, H,
                       (int)n, X, T, ldx, plan.tiles, plan.splits, plan.tok_per_split, plan.group,
                       part, counters);
  else
    hipLaunchKernelGGL(hess_bf16_kernel<true>, dim3((unsigned)grid), dim3(HTHREADS), 0, st, H,
                       (int)n, X, T, ldx, plan.tiles, plan.splits, plan.tok_per_split, plan.group,
                       part, counters);
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
