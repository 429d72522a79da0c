// Machine-peak probes for the roofline figures (measurement only; not part
// of the solver's C ABI, built into libsg_peaks.so).
//
//   sgp_mfma_bf16  chains of v_mfma_f32_16x16x32_bf16 on register operands
//   sgp_mfma_f32   chains of v_mfma_f32_16x16x4_f32 on register operands
//   sgp_copy       float4 grid-stride device copy (HBM read + write)
//   sgp_read       float4 grid-stride read with one sum per thread (HBM read)
//
// Each MFMA probe keeps eight independent accumulators per wave so that the
// matrix core never waits on a dependency, runs `iters` rounds of eight
// MFMAs, and stores the accumulators so that nothing is dead code.  The
// caller times the launch with events on `stream`.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float seed, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(lane + i));
    b[i] = (__bf16)(seed * (float)(lane - i));
  }
  floatx4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[u], 0, 0, 0);
  }
  floatx4 s = acc[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) s += acc[u];
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  out[t] = s[0] + s[1] + s[2] + s[3];
}

__global__ __launch_bounds__(256) void mfma_f32_kernel(int iters, float seed, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const float a = seed * (float)lane, b = seed * (float)(lane + 1);
  floatx4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[u], 0, 0, 0);
  }
  floatx4 s = acc[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) s += acc[u];
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  out[t] = s[0] + s[1] + s[2] + s[3];
}

__global__ __launch_bounds__(256) void copy_kernel(const floatx4* __restrict__ src, floatx4* __restrict__ dst,
                                                   int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_kernel(const floatx4* __restrict__ src, int64_t n4,
                                                   float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) s += src[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

extern "C" {

// out: blocks * 256 floats.  Work: blocks * 4 waves * iters * 8 MFMAs of
// 16 x 16 x 32 (bf16) or 16 x 16 x 4 (fp32), 2 flops per multiply-add.
int sgp_mfma_bf16(int iters, int blocks, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     1e-3f, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int sgp_mfma_f32(int iters, int blocks, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_f32_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     1e-3f, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// src, dst: n4 float4 each (16-byte aligned).
int sgp_copy(const void* src, void* dst, int64_t n4, int blocks, void* stream) {
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const floatx4*>(src), static_cast<floatx4*>(dst), n4);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// out: blocks * 256 floats.
int sgp_read(const void* src, int64_t n4, int blocks, float* out, void* stream) {
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const floatx4*>(src), n4, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
