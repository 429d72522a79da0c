// 2:4 compressed export of a pruned matrix: the kept values and a 2-bit
// position for each ("LLM 2:4 structured sparsity production guide", 2:4
// core-mechanism section: two of every four consecutive values along the
// reduction axis are kept, 2-bit metadata records their positions).
//
// One thread per 8 consecutive columns of a row (two groups of four): reads
// 32 bytes of W_hat and 8 mask bytes, writes four values and one metadata
// byte.  Neighbouring threads cover neighbouring columns, so every access of
// a wave is one contiguous span.  Purely HBM-bound: per element 4 + 1 bytes
// in, 2 (fp32) or 1 (bf16) + 1/8 bytes out.
#include "sg_internal.h"

#include <algorithm>

namespace sg {
namespace {

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float pick4(const float* v, unsigned i) {
  return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
}

// The two slots of a group from its kept bits (bit i set = position i kept):
// the kept positions in increasing order, then the pruned ones; the first two
// of that list, returned as i0 < i1.
__device__ __forceinline__ void group_slots(unsigned kept, unsigned& i0, unsigned& i1) {
  unsigned first = 4u, second = 4u;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (unsigned i = 0; i < 4; ++i) {
      const bool take = pass == 0 ? ((kept >> i) & 1u) : !((kept >> i) & 1u);
      if (take) {
        if (first == 4u) first = i;
        else if (second == 4u) second = i;
      }
    }
  }
  i0 = first < second ? first : second;
  i1 = first < second ? second : first;
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

template <bool VEC>
__global__ __launch_bounds__(256) void pack24_kernel(void* __restrict__ values, int v_dtype,
                                                     uint8_t* __restrict__ meta, int32_t* __restrict__ bad,
                                                     const float* __restrict__ W,
                                                     const uint8_t* __restrict__ mask, int64_t m,
                                                     int64_t n) {
  const int64_t per_row = (n + 7) >> 3;  // 8-column items = metadata bytes per row
  const int64_t items = m * per_row;
  const int64_t hn = n >> 1;             // values per row
  int nbad = 0;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * 256) {
    const int64_t r = it / per_row, q = it - r * per_row;
    const int64_t c0 = q * 8;
    const int ng = (n - c0 >= 8) ? 2 : 1;
    float w[8];
    unsigned kept = 0u;  // bit i: column c0 + i kept
    if (VEC) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(W + r * n + c0);
      const floatx4 b = *reinterpret_cast<const floatx4*>(W + r * n + c0 + 4);
      const uint64_t mk = *reinterpret_cast<const uint64_t*>(mask + r * n + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = a[e];
        w[4 + e] = b[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) kept |= (((mk >> (8 * e)) & 0xffull) == 0 ? 1u : 0u) << e;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = e < 4 * ng;
        const int64_t idx = r * n + c0 + (in ? e : 0);
        const bool k = in && mask[idx] == 0;
        w[e] = k ? W[idx] : 0.f;
        kept |= (k ? 1u : 0u) << e;
      }
    }
    float out[4];
    unsigned byte = 0u;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const unsigned kg = (kept >> (4 * g)) & 0xfu;
      unsigned i0, i1;
      group_slots(kg, i0, i1);
      const bool valid = g < ng;
      nbad += (valid && __popc(kg) > 2) ? 1 : 0;
      out[2 * g] = ((kg >> i0) & 1u) ? pick4(w + 4 * g, i0) : 0.f;
      out[2 * g + 1] = ((kg >> i1) & 1u) ? pick4(w + 4 * g, i1) : 0.f;
      if (valid) byte |= (i0 | (i1 << 2)) << (4 * g);
    }
    const int64_t vo = r * hn + 4 * q;
    if (v_dtype == SG_F32) {
      float* vf = static_cast<float*>(values);
      if (VEC) {
        *reinterpret_cast<floatx4*>(vf + vo) = floatx4{out[0], out[1], out[2], out[3]};
      } else {
        for (int e = 0; e < 2 * ng; ++e) vf[vo + e] = out[e];
      }
    } else {
      uint16_t* vb = static_cast<uint16_t*>(values);
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = to_bf16_rne(out[e]);
      if (VEC) {
        const uint64_t pk = (uint64_t)h[0] | ((uint64_t)h[1] << 16) | ((uint64_t)h[2] << 32) |
                            ((uint64_t)h[3] << 48);
        *reinterpret_cast<uint64_t*>(vb + vo) = pk;
      } else {
        for (int e = 0; e < 2 * ng; ++e) vb[vo + e] = h[e];
      }
    }
    meta[r * per_row + q] = static_cast<uint8_t>(byte);
  }
  if (nbad) atomicAdd(bad, nbad);
}

}  // namespace

sg_status launch_pack_two_four(void* values, int v_dtype, uint8_t* meta, int32_t* bad,
                               const float* W_hat, const uint8_t* mask, int64_t m, int64_t n,
                               hipStream_t st) {
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  const bool vec = (n % 8 == 0) && al(W_hat, 16) && al(mask, 8) &&
                   al(values, v_dtype == SG_F32 ? 16 : 8);
  const int64_t items = m * ((n + 7) >> 3);
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(items, 256), (int64_t)1 << 20);
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, st, bad);
  if (sg_status e = check_launch("pack 2:4 (clear)")) return e;
  if (vec)
    hipLaunchKernelGGL(pack24_kernel<true>, dim3(grid), dim3(256), 0, st, values, v_dtype, meta, bad,
                       W_hat, mask, m, n);
  else
    hipLaunchKernelGGL(pack24_kernel<false>, dim3(grid), dim3(256), 0, st, values, v_dtype, meta, bad,
                       W_hat, mask, m, n);
  return check_launch("pack 2:4");
}

}  // namespace sg
