// Hessian accumulation H += Xc^T Xc on gfx950.
//
// "SparseGPT ... Pruned in One-Shot" review (devpress), section 7: the layer's
// second-order information is H = X X^T of its calibration inputs.  X arrives
// token-major, Xc[t, c], so H[i][j] = sum_t Xc[t][i] Xc[t][j]: a symmetric
// rank-T update whose reduction axis (tokens) is the strided one.
//
// bf16 path: output tiles of 256 rows x 384 columns covering the lower
// triangle (row panel I takes the column panels that reach its last row; the
// symmetric result is mirrored on store), 8 waves per workgroup, each wave a
// 128x96 sub-tile of v_mfma_f32_16x16x32_bf16 (two waves per SIMD, 192
// accumulators a lane).  Token rows are copied as they lie in X straight from
// global memory into LDS by the LDS-DMA loads, and the operands are gathered
// by the transposing LDS read.  Rows are read in 16-byte chunks up to n
// rounded up to 8 channels (inside the row: the ABI asks for ldx % 8 == 0);
// channels past n only feed outputs past n, which are never stored.
// When there are too few tiles to fill the 256 CUs the tokens are split; every
// split writes its partial tile to the workspace and the last split to finish
// sums all partials in split order (bitwise reproducible), then adds into H.
//
// Tile order: the hardware deals workgroups round-robin over the 8 XCDs, each
// with its own L2.  Tiles are enumerated in g x g groups of panels (row panel
// = 256 channels, column panel = 384), and XCD x takes a contiguous eighth of
// that order, split-major: the workgroups resident on one XCD then work on a
// compact set of tiles that share few panels, over the same token range, so X
// re-reads can hit its L2; the XCDs run the same token range at the same time,
// which the shared Infinity Cache serves once.
// Lockstep: left alone, the 32 workgroups of one XCD drift apart by far more
// tokens than its 4 MB L2 holds, and only about one X read in six hits there
// (measured at n = 28672).  Each "round" of 32 workgroups of an XCD (those
// that start together, on one token split) therefore shares a progress
// counter: every 32 stages
// a workgroup adds one, and before the next 32 it waits until all of its
// round have finished the previous ones.  With that, three reads in four hit
// the L2 and the fabric traffic falls threefold.  The wait is bounded: a
// workgroup that polls too long (peers not resident, say, because another
// kernel holds CUs) stops waiting for the rest of its tile; the counters
// order nothing that the result depends on.
#include "sg_internal.h"

#include <math.h>

#include <algorithm>
#include <functional>

namespace sg {
namespace {

constexpr int HTI = kHessTileRows;     // 256
constexpr int HTJ = kHessTileCols;     // 384
constexpr int HSPLIT_ALIGN = 64;     // tokens: split boundaries are multiples of this
constexpr int HTHREADS = 512;
constexpr int kMinTokPerSplit = 4096;
// A workgroup's fixed cost in tokens' worth of its time: 3,700 for 256x256
// tiles (measured at n = 4096, 262,144 tokens: 15 equal splits were 3%
// slower than 7), scaled by the 1.5x work per token of a 256x384 tile
constexpr int kWgCostTok = 2500;
constexpr int kCuPerXcd = kNumCU / 8;  // workgroups of one lockstep round
constexpr int kSyncEvery = 8;          // steady-state iterations (4 stages each) per counter step
constexpr int kSyncSpin = 400;         // polls before a workgroup stops waiting

// ti-th tile (I, J), J <= I, of a lower triangle of square tiles, row-major.
__device__ inline void tri_decode(int64_t ti, int& I, int& J) {
  int64_t r = (int64_t)((sqrt(8.0 * (double)ti + 1.0) - 1.0) * 0.5);
  while ((r + 1) * (r + 2) / 2 <= ti) ++r;
  while (r * (r + 1) / 2 > ti) --r;
  I = (int)r;
  J = (int)(ti - r * (r + 1) / 2);
}

// Column panels of row panel I: those holding a column <= its last row.
__host__ __device__ inline int tile_cols(int I, int n) {
  const int r = min(n - 1, I * HTI + HTI - 1);
  return r / HTJ + 1;
}

// k-th tile of the grouped order: row panels in blocks of g; inside a block,
// the column panels in groups of g, and inside a group the block's rows one
// after another, each with its columns of the group.
__host__ __device__ inline void tile_decode(int64_t k, int n, int g, int& I, int& J) {
  const int nI = (n + HTI - 1) / HTI;
  I = 0;
  J = 0;
  for (int r0 = 0; r0 < nI; r0 += g) {
    const int gi = min(g, nI - r0);
    int64_t blk = 0;
    int maxJ = 0;
    for (int i = 0; i < gi; ++i) {
      const int c = tile_cols(r0 + i, n);
      blk += c;
      maxJ = max(maxJ, c);
    }
    if (k >= blk) {
      k -= blk;
      continue;
    }
    for (int c0 = 0; c0 < maxJ; c0 += g) {
      int64_t grp = 0;
      for (int i = 0; i < gi; ++i) grp += min(g, max(0, tile_cols(r0 + i, n) - c0));
      if (k >= grp) {
        k -= grp;
        continue;
      }
      for (int i = 0; i < gi; ++i) {
        const int w = min(g, max(0, tile_cols(r0 + i, n) - c0));
        if (k < w) {
          I = r0 + i;
          J = c0 + (int)k;
          return;
        }
        k -= w;
      }
    }
  }
}

__global__ void zero_u32_kernel(unsigned* p, int64_t cnt) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < cnt) p[i] = 0u;
}

// The X stages are copied straight from global memory into LDS by the
// LDS-DMA loads (no register staging, no transposes in VALU).  A stage is 32
// tokens; in LDS each token is one 1280-byte row holding the tile's row panel
// (256 channels) and column panel (384 channels), 80 chunks of 16 bytes.  Rows
// are not padded (four stages fill the 160 KB): instead chunk p of token row
// t holds the row's chunk p ^ 2 tau(t), tau(t) = (t & 3) | ((t & 8) >> 1), a
// swap of whole 32-byte pairs inside aligned 256-byte groups, so that the 8
// token rows one half-wave of a transposing read touches (t = 0..3 and 8..11,
// or 4..7 and 12..15, plus 16) fall on 8 different bank groups.
// MFMA operands (8 consecutive tokens of one channel per lane) are read with
// the transposing LDS read, which gathers 4 tokens x 4 channels across 16
// lanes.  Four stages rotate, three in flight while the fourth is multiplied.
constexpr int DK = 32;                       // tokens per stage
constexpr int DROW = (HTI + HTJ) * 2;        // 1280 LDS bytes per token row
constexpr int DCH = DROW / 16;               // 80 chunks per token row
constexpr int DSTAGE = DK * DROW;            // 40960 bytes per stage
constexpr int kNB = 6;                       // 16-column fragments of a wave's 96 columns

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// s_waitcnt immediates that wait for the vector-memory counter only (a wave
// issues 5 copies per stage).
constexpr unsigned kWaitVm0 = 0x0F70u;
constexpr unsigned kWaitVm5 = 0x0F75u;
constexpr unsigned kWaitVm10 = 0x0F7Au;

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
    int64_t ldx, int64_t tiles, int splits, const HessSplits bounds, int group,
    float* __restrict__ part, unsigned* __restrict__ counters, unsigned* __restrict__ sync,
    int sync_rounds) {
  // One array per stage (together the whole 160 KB).
  __shared__ __attribute__((aligned(16))) unsigned char st0[DSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[DSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[DSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st3[DSTAGE];

  const int xcd = blockIdx.x & 7;
  const int64_t jx = blockIdx.x >> 3;
  const int64_t k0 = tiles * xcd / 8, k1 = tiles * (xcd + 1) / 8;
  const int64_t cnt = k1 - k0;
  if (jx >= cnt * splits) return;
  const int split = (int)(jx / cnt);
  const int64_t ti = k0 + (jx - (int64_t)split * cnt);
  const int64_t item = (int64_t)split * tiles + ti;
  int I, J;
  tile_decode(ti, n, group, I, J);
  const int i0 = I * HTI, j0 = J * HTJ;
  const int64_t t_begin = bounds.b[split];
  const int64_t t_end = min(T, bounds.b[split + 1]);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wi = wave >> 2;
  const int wj = wave & 3;

  floatx4 acc[8][kNB];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < kNB; ++c) acc[a][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Copy role: wave w fills token rows 4w..4w+3 of every stage, 320 chunks in
  // 5 instructions of 64 lanes (lane l of instruction k writes LDS chunk
  // 64k + l of those rows, so it reads row r = (64k + l) / 80, chunk
  // p ^ 2 tau with p = (64k + l) % 80).  Chunks past n8 (n rounded up to 8,
  // still inside the row since ldx is a multiple of 8) re-read the last chunk:
  // channels past n only feed outputs beyond n, which are never stored.
  const int n8 = (n + 7) & ~7;
  auto chunk_src = [&](int idx, int& r) {
    r = idx / DCH;
    const int p = idx - r * DCH;
    const int g = p ^ (2 * (r | ((wave & 2) << 1)));  // tau of token row 4 wave + r
    const int col = g < 32 ? i0 + 8 * g : j0 + 8 * (g - 32);
    return col < n8 ? col : n8 - 8;
  };
  uint32_t voff[5];  // the host keeps 4 * ldx * 2 bytes below 2^31
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    int r;
    const int col = chunk_src(64 * k + lane, r);
    voff[k] = (uint32_t)((int64_t)r * ldx * 2 + (int64_t)col * 2);
  }
  // every stage but the last is full
  auto copy_full = [&](unsigned char* buf, int64_t s) {
    const int64_t tok0 = t_begin + s * DK + wave * 4;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)buf + (uint32_t)(wave * 4 * DROW);
    const char* base = reinterpret_cast<const char*>(X) + tok0 * ldx * 2;
#pragma unroll
    for (int k = 0; k < 5; ++k)
      lds_dma16(base, voff[k], __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(k * 1024)));
  };
  // any stage: token rows past the end re-read the last row (zeroed before use)
  auto copy_stage = [&](unsigned char* buf, int64_t s) {
    const int64_t tok0 = t_begin + s * DK + wave * 4;
    if (tok0 + 3 < t_end) {
      copy_full(buf, s);
      return;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)buf + (uint32_t)(wave * 4 * DROW);
    const int64_t rmax = t_end - 1 - tok0;
    const int64_t tb = rmax >= 0 ? tok0 : t_end - 1;
    const char* base = reinterpret_cast<const char*>(X) + tb * ldx * 2;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      int r;
      const int col = chunk_src(64 * k + lane, r);
      const int64_t re = rmax >= 0 ? min<int64_t>(r, rmax) : 0;
      lds_dma16(base, (uint32_t)(re * ldx * 2 + (int64_t)col * 2),
                __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(k * 1024)));
    }
  };

  // Operand addresses: lane l of a transposing read points at token row
  // trow = 8*(l/16) + (l%16)/4 (+4 for the second read, same tau) and channel
  // quad l%4 of the 16-channel fragment; lane i of the result then holds
  // channel i of the fragment over those 4 tokens.  Fragment a of the row
  // panel is pair 8 wi + a of the row, fragment c of the column panel pair
  // 16 + 6 wj + c; the swizzle moves pair q to q ^ tau.
  const int s16 = lane & 15;
  const int trow = 8 * (lane >> 4) + (s16 >> 2);
  int tau = (trow & 3) | ((trow & 8) >> 1);
  const int hq = s16 & 3;
  uint32_t lbase = (uint32_t)(trow * DROW + (hq >> 1) * 16 + (hq & 1) * 8);
  auto a_off = [&](int a) { return lbase + 32u * (uint32_t)(8 * wi + (a ^ tau)); };
  auto b_off = [&](int c) { return lbase + 32u * (uint32_t)((16 + 6 * wj + c) ^ tau); };

  auto frag = [&](const unsigned char* buf, uint32_t off) {
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(buf + off));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(buf + off + 4 * DROW));
    const shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  };

  auto compute = [&](const unsigned char* buf) {
    bf16x8 fb[kNB];
#pragma unroll
    for (int c = 0; c < kNB; ++c) fb[c] = frag(buf, b_off(c));
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const bf16x8 fa = frag(buf, a_off(a));
#pragma unroll
      for (int c = 0; c < kNB; ++c)
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
  // multiply stage s with each row-panel fragment read one ahead of its
  // products, and read the first fragments of stage s+1 after the last
  // products that use the current ones (192 accumulators leave no room to
  // hold both sets).
  struct Frags {
    bf16x8 fb[kNB];
    bf16x8 fa0;
  };
  auto prefetch = [&](const unsigned char* buf, Frags& f) {
#pragma unroll
    for (int c = 0; c < kNB; ++c) f.fb[c] = frag(buf, b_off(c));
    f.fa0 = frag(buf, a_off(0));
  };
  auto step = [&](const unsigned char* cur, const unsigned char* nxt, unsigned char* refill,
                  int64_t s, Frags& f) {
    __builtin_amdgcn_s_waitcnt(kWaitVm5);
    stage_barrier();
    copy_full(refill, s + 3);
    __builtin_amdgcn_sched_barrier(0);
    // the swizzled operand addresses are recomputed every step rather than
    // held in registers across the loop
    asm volatile("" : "+v"(tau), "+v"(lbase));
    bf16x8 fa = f.fa0;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const bf16x8 fan = a < 7 ? frag(cur, a_off(a + 1)) : frag(nxt, a_off(0));
#pragma unroll
      for (int c = 0; c < kNB; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f.fb[c], acc[a][c], 0, 0, 0);
      fa = fan;
    }
    f.fa0 = fa;
#pragma unroll
    for (int c = 0; c < kNB; ++c) f.fb[c] = frag(nxt, b_off(c));
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int g = 0; g < 7; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, kNB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kNB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kNB, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Lockstep counter of this workgroup's group: the workgroups of its round
  // (32 consecutive ones of the XCD) that work on the same token split.
  // Thread 0 alone touches it.
  const int64_t round = jx / kCuPerXcd;
  const int64_t g0 = max<int64_t>(round * kCuPerXcd, (int64_t)split * cnt);
  const int64_t g1 = min<int64_t>((round + 1) * kCuPerXcd, (int64_t)(split + 1) * cnt);
  const int64_t active = g1 - g0;
  unsigned* const my_sync =
      sync ? sync + ((int64_t)xcd * sync_rounds + round) * splits + split : nullptr;
  bool waiting = true;
  int64_t s = 0;
  if (nsteps > 6) {
    __builtin_amdgcn_s_waitcnt(kWaitVm5);  // stages 0 and 1
    stage_barrier();
    Frags f;
    prefetch(st0, f);
    for (; s + 6 < nsteps; s += 4) {
      const int64_t it = s >> 2;
      if (my_sync && tid == 0 && waiting && it > 0 && it % kSyncEvery == 0) {
        // the other waves wait for this one at the next stage barrier
        const int64_t need = (it / kSyncEvery) * active;
        int k = 0;
        for (; k < kSyncSpin; ++k) {
          if ((int64_t)__hip_atomic_load(my_sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) break;
          __builtin_amdgcn_s_sleep(2);
        }
        if (k == kSyncSpin) waiting = false;
      }
      step(st0, st1, st3, s, f);
      step(st1, st2, st0, s + 1, f);
      step(st2, st3, st1, s + 2, f);
      step(st3, st0, st2, s + 3, f);
      if (my_sync && tid == 0 && (it + 1) % kSyncEvery == 0)
        __hip_atomic_fetch_add(my_sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  for (; s < nsteps; ++s) {
    const int b = (int)(s & 3);
    unsigned char* cur = b == 0 ? st0 : b == 1 ? st1 : b == 2 ? st2 : st3;
    unsigned char* refill = b == 0 ? st3 : b == 1 ? st0 : b == 2 ? st1 : st2;
    const int64_t later = nsteps - 1 - s;
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(kWaitVm10);
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(kWaitVm5);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stage_barrier();
    const int valid = (int)min<int64_t>(DK, ntok - s * DK);
    if (valid < DK) {
      // last, partial stage: zero the token rows past the end
      for (int e = tid; e < (DK - valid) * DCH; e += HTHREADS) {
        const int row = valid + e / DCH;
        *reinterpret_cast<u32x4*>(cur + row * DROW + (e % DCH) * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (s + 3 < nsteps) copy_stage(refill, s + 3);
    compute(cur);
  }

  // ---- epilogue -----------------------------------------------------------
  // Row fragment a of the wave's sub-tile (16 rows x 96 columns, held as
  // kNB float4 per lane) added into H's lower triangle, and mirrored (tiles
  // that cross the diagonal hold upper entries too, which the mirror of the
  // lower ones writes).
  auto store_frag = [&](int a, const floatx4 (&v4)[kNB]) {
#pragma unroll
    for (int c = 0; c < kNB; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i0 + wi * 128 + a * 16 + (lane >> 4) * 4 + v;
        const int col2 = j0 + wj * 96 + c * 16 + (lane & 15);
        if (row >= n || col2 >= n || row < col2) continue;
        const size_t lo = (size_t)row * n + col2;
        const float val = H[lo] + v4[c][v];
        H[lo] = val;
        if (row != col2) H[(size_t)col2 * n + row] = val;
      }
  };
  // Token splits: each split writes its partial tile (per (wave, a, c) slot,
  // 64 lanes x float4); the last split to arrive sums every partial in split
  // order (its own re-read too, so the result does not depend on which split
  // finished last) and adds into H.
  if (splits > 1) {
    floatx4* mine = reinterpret_cast<floatx4*>(part + (size_t)item * (HTI * HTJ));
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < kNB; ++c) mine[(wave * 8 * kNB + a * kNB + c) * 64 + lane] = acc[a][c];
    __threadfence();
    __syncthreads();
    // every wave is past its last read of the stages: the flag uses stage 0
    int* const s_last = reinterpret_cast<int*>(st0);
    if (tid == 0) {
      const unsigned old = atomicAdd(&counters[ti], 1u);
      *s_last = (old == (unsigned)(splits - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!*s_last) return;
    __threadfence();
    // The register tile is not needed any more (this split's partial is read
    // back like the others), so the registers hold loads instead: for each
    // row fragment, the slots of up to eight splits are requested together
    // (a serial sum with few loads in flight was bound by their latency).
    constexpr int SG = 8;
    const floatx4* const base = reinterpret_cast<const floatx4*>(part + (size_t)ti * (HTI * HTJ));
    const size_t sstride = (size_t)tiles * (HTI * HTJ / 4);  // float4 between splits of a tile
    for (int a = 0; a < 8; ++a) {
      floatx4 sum[kNB];
      const floatx4* slot = base + (size_t)(wave * 8 * kNB + a * kNB) * 64 + lane;
      for (int sp0 = 0; sp0 < splits; sp0 += SG) {
        floatx4 pv[SG][kNB];
#pragma unroll
        for (int q = 0; q < SG; ++q)
          if (sp0 + q < splits) {
#pragma unroll
            for (int c = 0; c < kNB; ++c) pv[q][c] = slot[(size_t)(sp0 + q) * sstride + c * 64];
          }
#pragma unroll
        for (int q = 0; q < SG; ++q)
          if (sp0 + q < splits) {
#pragma unroll
            for (int c = 0; c < kNB; ++c) sum[c] = (sp0 + q == 0) ? pv[q][c] : sum[c] + pv[q][c];
          }
      }
      store_frag(a, sum);
    }
    if (tid == 0) counters[ti] = 0u;
    return;
  }

#pragma unroll
  for (int a = 0; a < 8; ++a) store_frag(a, acc[a]);
}

// fp32 inputs: 64x64 lower-triangle tiles on v_mfma_f32_16x16x4_f32.  A
// 32-token stage of both 64-channel panels sits in LDS as it lies in X
// (token rows, channels contiguous); each of the 4 waves owns a 32x32
// sub-tile (2x2 MFMA blocks), and lane l reads its operand value (channel
// l % 16 of a block, token l / 16 of a 4-token step) straight from a token
// row, so consecutive lanes read consecutive words.  Each stage is summed in
// its own accumulators before it is added to the running total (32-token
// partial sums): fp32 products, unlike bf16 ones, are rounded.
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
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  floatx4 tot[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) tot[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  // loader: thread t stages channel t % 64 of token rows t / 64 + 4 u
  const int lc = tid & 63, lr = tid >> 6;
  const bool aok = i0 + lc < n, bok = j0 + lc < n;
  const int64_t ca = aok ? i0 + lc : n - 1, cb = bok ? j0 + lc : n - 1;
  for (int64_t t0 = 0; t0 < T; t0 += FBK) {
    float va[FBK / 4], vb[FBK / 4];
#pragma unroll
    for (int u = 0; u < FBK / 4; ++u) {
      const int64_t t = t0 + lr + 4 * u;
      const int64_t tc = t < T ? t : T - 1;  // clamped in-bounds address, zeroed below
      va[u] = X[tc * ldx + ca];
      vb[u] = X[tc * ldx + cb];
    }
#pragma unroll
    for (int u = 0; u < FBK / 4; ++u) {
      const bool tok = t0 + lr + 4 * u < T;
      As[lr + 4 * u][lc] = (tok && aok) ? va[u] : 0.f;
      Bs[lr + 4 * u][lc] = (tok && bok) ? vb[u] : 0.f;
    }
    __syncthreads();
    floatx4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < FBK; k += 4) {
      const int kr = k + (lane >> 4);
      float fa[2], fb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) fa[a] = As[kr][wi * 32 + a * 16 + (lane & 15)];
#pragma unroll
      for (int b = 0; b < 2; ++b) fb[b] = Bs[kr][wj * 32 + b * 16 + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) tot[a][b] += acc[a][b];
    __syncthreads();
  }
  // lane l, register v of block (a, b): row 4 (l / 16) + v, column l % 16
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i0 + wi * 32 + a * 16 + (lane >> 4) * 4 + v;
        const int col = j0 + wj * 32 + b * 16 + (lane & 15);
        if (row >= n || col >= n) continue;
        if (I == J && row < col) continue;
        const size_t lo = (size_t)row * n + col;
        const float val = H[lo] + tot[a][b][v];
        H[lo] = val;
        if (row != col) H[(size_t)col * n + row] = val;
      }
}

}  // namespace

// Finish time of one XCD's share (per_xcd tiles of every split, split-major,
// each workgroup to the first of its CUs that is free) in units of the time
// one workgroup takes for all T tokens; c_wg: a workgroup's fixed cost
// (pipeline fill, partial tile, the last split's sum) in the same unit.
double split_makespan(const double* frac, int nfrac, int64_t per_xcd, double c_wg) {
  double cu[kCuPerXcd] = {};  // min-heap of the CUs' finish times
  for (int s = 0; s < nfrac; ++s)
    for (int64_t t = 0; t < per_xcd; ++t) {
      std::pop_heap(cu, cu + kCuPerXcd, std::greater<double>());
      cu[kCuPerXcd - 1] += frac[s] + c_wg;
      std::push_heap(cu, cu + kCuPerXcd, std::greater<double>());
    }
  return *std::max_element(cu, cu + kCuPerXcd);
}

HessPlan hessian_plan(int64_t n, int64_t T, size_t ws_avail, bool limit_by_ws) {
  HessPlan p{};
  const int64_t nI = ceil_div(n, HTI);
  p.tiles = 0;
  for (int I = 0; I < nI; ++I) p.tiles += tile_cols(I, (int)n);
  const size_t tile_bytes = (size_t)HTI * HTJ * sizeof(float);
  const size_t cnt_bytes = round_up(p.tiles * sizeof(unsigned), 256);
  int max_s = (int)std::max<int64_t>(1, std::min<int64_t>(kHessMaxSplits, T / kMinTokPerSplit));
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
  // Measured at n = 4096, T = 262144 with 256x256 tiles: 7 splits (4
  // rounds, 93% full) take 4.50-4.60 ms, 15 splits (8 rounds, 99.6% full)
  // 4.63-4.73 ms.
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
  // Equal splits, then (when the tokens are split at all) unequal ones if a
  // simulated schedule finishes sooner: big splits first, a few smaller
  // ones last to fill the tail of the last round.  Measured at n = 4096,
  // T = 262144 with 256x256 tiles: three splits of 28% and two of 8% take
  // 4.37 ms against 4.55-4.67 ms for 7 equal ones.
  double frac[kHessMaxSplits];
  int nfrac = best_s;
  for (int s = 0; s < best_s; ++s) frac[s] = 1.0 / best_s;
  if (best_s > 1) {
    const int64_t per_xcd = ceil_div(p.tiles, 8);
    const double c_wg = (double)kWgCostTok / (double)T;
    double best_ms = split_makespan(frac, nfrac, per_xcd, c_wg);
    double cand[kHessMaxSplits];
    for (int k = std::max(1, best_s - 5); k <= best_s + 1 && k < max_s; ++k)
      for (int j = 1; j <= 2 && k + j <= max_s; ++j)
        for (int r = 2; r <= 4; ++r) {
          // k splits of size a, j of size a * r / 10
          const double a = 1.0 / (k + j * r / 10.0), b = a * r / 10.0;
          if (b * (double)T < (double)kMinTokPerSplit) continue;
          for (int s = 0; s < k + j; ++s) cand[s] = s < k ? a : b;
          const double ms = split_makespan(cand, k + j, per_xcd, c_wg);
          if (ms < best_ms * 0.98) {
            best_ms = ms;
            nfrac = k + j;
            std::copy(cand, cand + nfrac, frac);
          }
        }
  }
  p.bounds.b[0] = 0;
  int ns = 0;
  double acc = 0.0;
  for (int s = 0; s < nfrac && p.bounds.b[ns] < T; ++s) {
    acc += frac[s];
    const int64_t e = s + 1 == nfrac ? T : std::min<int64_t>(T, round_up((int64_t)(acc * (double)T), HSPLIT_ALIGN));
    if (e > p.bounds.b[ns]) p.bounds.b[++ns] = e;
  }
  if (ns == 0 || p.bounds.b[ns] < T) p.bounds.b[++ns] = T;  // (no tokens: one empty split)
  p.splits = ns;
  p.part_bytes = p.splits > 1 ? cnt_bytes + tile_bytes * (size_t)p.tiles * p.splits : 0;
  // Lockstep counters (8 XCDs x rounds x splits), after the partials, when
  // the tokens are not split.  With splits, groups of one split per round
  // were measured too (n = 4096, 7 splits): no gain, the tiles of a split
  // already share their panels in L2 at about the rate the counters give.
  // Without room for the counters in the workspace the launch runs
  // unsynchronised (same result, more fabric traffic).
  p.sync_rounds = (int)ceil_div(ceil_div(p.tiles, 8) * p.splits, kCuPerXcd);
  const size_t sync_bytes =
      p.splits == 1 ? round_up((int64_t)8 * p.sync_rounds * p.splits * sizeof(unsigned), 256) : 0;
  p.ws_bytes = p.part_bytes + sync_bytes;
  p.sync = sync_bytes > 0 && (!limit_by_ws || ws_avail >= p.ws_bytes);
  // Group edge: about the square root of the tiles an XCD has resident at once
  // (its 32 CUs, or its whole share when that is smaller).
  const double per_xcd = std::min<double>(32.0, (double)p.tiles * p.splits / 8.0) /
                         std::max(1, std::min(p.splits, 2));
  p.group = (int)std::max<int64_t>(1, std::min<int64_t>(nI, (int64_t)std::lround(std::sqrt(per_xcd))));
  p.grid = 8 * ceil_div(p.tiles, 8) * p.splits;
  return p;
}

sg_status launch_hessian_bf16(float* H, int64_t n, const uint16_t* X, int64_t T,
                              int64_t ldx, const HessPlan& plan, void* ws,
                              hipStream_t st) {
  unsigned* counters = nullptr;
  float* part = nullptr;
  unsigned* sync = nullptr;
  if (plan.splits > 1) {
    counters = reinterpret_cast<unsigned*>(ws);
    part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                    round_up(plan.tiles * sizeof(unsigned), 256));
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)ceil_div(plan.tiles, 256)), dim3(256),
                       0, st, counters, plan.tiles);
    if (sg_status e = check_launch("hessian counters")) return e;
  }
  if (plan.sync) {
    const int64_t cnt = (int64_t)8 * plan.sync_rounds * plan.splits;
    sync = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + plan.part_bytes);
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)ceil_div(cnt, 256)), dim3(256), 0, st, sync, cnt);
    if (sg_status e = check_launch("hessian lockstep counters")) return e;
  }
  const int64_t grid = plan.grid;
  hipLaunchKernelGGL(hess_bf16_dma_kernel, dim3((unsigned)grid), dim3(HTHREADS), 0, st, H,
                     (int)n, X, T, ldx, plan.tiles, plan.splits, plan.bounds, plan.group,
                     part, counters, sync, plan.sync_rounds);
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
