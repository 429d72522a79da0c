// Internal declarations of the gfx950 SparseGPT layer solver library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sg.h"
#include "hessian.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNumCU = 256;       // MI355X compute units (launch sizing only)
constexpr int kFactorNB = 128;    // factorisation panel width
constexpr int kGemmTile = 128;    // fp32 MFMA update tile edge
constexpr int kSelBins = 2048;    // radix-select histogram bins
constexpr int kRecTile = 128;     // reconstruction-error output tile edge

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

__device__ inline float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// ---------------------------------------------------------------------------
// Host-side error reporting (thread-local message).
// ---------------------------------------------------------------------------
sg_status set_error(sg_status s, const char* fmt, ...);
sg_status check_launch(const char* what);

// ---------------------------------------------------------------------------
// Factorisation
// ---------------------------------------------------------------------------
size_t factor_ws_bytes(int64_t n);
sg_status launch_prepare_hinv(float* Hinv, const float* H, int64_t n, double damp,
                              int32_t* info, void* ws, hipStream_t st, hipStream_t side,
                              hipEvent_t ev_a, hipEvent_t ev_b);
// nl layers of order n in one set of launches; layer L's part of the workspace
// starts factor_ws_bytes(n) * L bytes in; info[L] is its status.
sg_status launch_prepare_hinv_batched(float* const* Hinv, const float* const* H, int nl, int64_t n,
                                      double damp, int32_t* info, void* ws, hipStream_t st,
                                      hipStream_t side, hipEvent_t ev_a, hipEvent_t ev_b);

// ---------------------------------------------------------------------------
// Prune
// ---------------------------------------------------------------------------
struct PruneArgs {
  float* W_out;
  uint8_t* mask_out;
  const void* W;
  int w_dtype;
  int64_t m, n, ldw;
  const float* U;
  // seg_u: every stacked matrix has a factor of its own, Useg[p] (else all
  // share U)
  bool seg_u;
  const float* Useg[SG_MAX_SEGMENTS];
  int kind;
  double sparsity;
  int n_keep, m_group;
  int blocksize;
  const uint8_t* mask_in;
  // row segments: W stacks nseg matrices that share the input (and U);
  // unstructured selection is per segment
  int nseg;
  int64_t seg_rows[SG_MAX_SEGMENTS + 1];
  // vector-level removal: 1 = column by column, 16 = joint per 16 columns
  int vec;
  // joint quantization (bits == 0: pruning only)
  int bits;
  uint8_t* codes_out;
  float* qscale;
  float* qzero;
};
size_t prune_ws_bytes(int64_t m, int64_t n, int blocksize);
// The no-allocation prune entry point's scratch array (per device; its size
// is SG_NOALLOC_SCRATCH_BYTES): its device address on the current device.
constexpr size_t kNoAllocScratchBytes = SG_NOALLOC_SCRATCH_BYTES;
sg_status noalloc_scratch(void** ptr);
sg_status launch_prune(const PruneArgs& a, void* ws, hipStream_t st);

// ---------------------------------------------------------------------------
// 2:4 compressed export
// ---------------------------------------------------------------------------
sg_status launch_pack_two_four(void* values, int v_dtype, uint8_t* meta, int32_t* bad,
                               const float* W_hat, const uint8_t* mask, int64_t m, int64_t n,
                               hipStream_t st);

// ---------------------------------------------------------------------------
// Reconstruction error
// ---------------------------------------------------------------------------
size_t recon_ws_bytes(int64_t m, int64_t T);
sg_status launch_recon(double* err, int accumulate, const void* W, int w_dtype,
                       int64_t ldw, const float* W_hat, int64_t m, int64_t n,
                       const void* X, int x_dtype, int64_t T, int64_t ldx,
                       void* ws, hipStream_t st);

}  // namespace sg
