// C ABI entry points: argument validation, workspace carving, gfx950 check.
// Every host-detectable problem is reported before anything is enqueued.
#include "sg_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

namespace sg {

static thread_local std::string g_last_error;

sg_status set_error(sg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sg_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(SG_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return SG_OK;
}

namespace {

constexpr int kMaxDev = 64;
std::mutex g_dev_mu;
int g_dev_ok[kMaxDev];  // 0 unknown, 1 gfx950, -1 other

sg_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return set_error(SG_ERR_HIP, "no current HIP device");
  if (dev >= kMaxDev) return set_error(SG_ERR_UNSUPPORTED, "device index %d too large", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return set_error(SG_ERR_HIP, "hipGetDeviceProperties failed");
    g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  if (g_dev_ok[dev] != 1)
    return set_error(SG_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X/MI350X)", dev);
  return SG_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace
}  // namespace sg

using namespace sg;

extern "C" {

int32_t sg_abi_version(void) { return SG_ABI_VERSION; }

const char* sg_status_string(sg_status s) {
  switch (s) {
    case SG_OK: return "SG_OK";
    case SG_ERR_INVALID_ARGUMENT: return "SG_ERR_INVALID_ARGUMENT";
    case SG_ERR_UNSUPPORTED: return "SG_ERR_UNSUPPORTED";
    case SG_ERR_WORKSPACE: return "SG_ERR_WORKSPACE";
    case SG_ERR_HIP: return "SG_ERR_HIP";
    default: return "SG_ERR_UNKNOWN";
  }
}

const char* sg_last_error_message(void) { return g_last_error.c_str(); }

size_t sg_workspace_bytes(int32_t op, int64_t m, int64_t n, int64_t T, int32_t blocksize) {
  switch (op) {
    case SG_OP_HESSIAN:
      if (n < 1 || T < 1) return 0;
      return hessian_plan(n, T, 0, false).ws_bytes;
    case SG_OP_PREPARE_HINV:
      if (n < 1) return 0;
      return factor_ws_bytes(n);
    case SG_OP_PRUNE:
      if (m < 1 || n < 1 || blocksize < 1 || blocksize > SG_MAX_BLOCKSIZE) return 0;
      return prune_ws_bytes(m, n, blocksize);
    case SG_OP_RECON:
      if (m < 1 || n < 1 || T < 1) return 0;
      return recon_ws_bytes(m, T);
    default:
      return 0;
  }
}

sg_status sg_hessian_accumulate(float* H, int64_t n, const void* X, int32_t x_dtype, int64_t T,
                                int64_t ldx, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!H || !X) return set_error(SG_ERR_INVALID_ARGUMENT, "H and X must not be NULL");
  if (n < 1 || n > 65536) return set_error(SG_ERR_INVALID_ARGUMENT, "n=%lld out of [1, 65536]", (long long)n);
  if (T < 1) return set_error(SG_ERR_INVALID_ARGUMENT, "T=%lld must be >= 1", (long long)T);
  if (ldx < n) return set_error(SG_ERR_INVALID_ARGUMENT, "ldx=%lld < n=%lld", (long long)ldx, (long long)n);
  if (x_dtype != SG_BF16 && x_dtype != SG_F32)
    return set_error(SG_ERR_UNSUPPORTED, "x_dtype %d not supported", x_dtype);
  if (x_dtype == SG_BF16 && (!aligned(X, 16) || (ldx % 8) != 0))
    return set_error(SG_ERR_UNSUPPORTED, "bf16 X must be 16-byte aligned with ldx %% 8 == 0");
  if (x_dtype == SG_BF16 && ldx >= ((int64_t)1 << 28))
    return set_error(SG_ERR_UNSUPPORTED, "bf16 X rows must lie fewer than 2^28 elements apart");
  if (ws_bytes > 0 && !workspace)
    return set_error(SG_ERR_INVALID_ARGUMENT, "workspace is NULL but ws_bytes > 0");
  if (workspace && !aligned(workspace, 256))
    return set_error(SG_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (sg_status e = check_device()) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (x_dtype == SG_BF16) {
    const HessPlan plan = hessian_plan(n, T, workspace ? ws_bytes : 0, true);
    return launch_hessian_bf16(H, n, static_cast<const uint16_t*>(X), T, ldx, plan, workspace, st);
  }
  return launch_hessian_f32(H, n, static_cast<const float*>(X), T, ldx, st);
}

sg_status sg_prepare_hinv(float* Hinv, const float* H, int64_t n, double damp, int32_t* info,
                          void* workspace, size_t ws_bytes, void* stream, void* update_stream,
                          void* event_a, void* event_b) {
  g_last_error.clear();
  if (!Hinv || !H || !info) return set_error(SG_ERR_INVALID_ARGUMENT, "Hinv, H and info must not be NULL");
  if (n < 1 || n > 65536) return set_error(SG_ERR_INVALID_ARGUMENT, "n=%lld out of [1, 65536]", (long long)n);
  if (!(damp >= 0.0) || !isfinite(damp))
    return set_error(SG_ERR_INVALID_ARGUMENT, "damp must be finite and >= 0");
  if (static_cast<const void*>(Hinv) == static_cast<const void*>(H))
    return set_error(SG_ERR_INVALID_ARGUMENT, "Hinv must not alias H");
  const size_t need = factor_ws_bytes(n);
  if (!workspace || ws_bytes < need)
    return set_error(SG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned(workspace, 256))
    return set_error(SG_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const int given = (update_stream != nullptr) + (event_a != nullptr) + (event_b != nullptr);
  if (given != 0 && given != 3)
    return set_error(SG_ERR_INVALID_ARGUMENT, "update_stream, event_a and event_b go together (all or none)");
  if (given == 3 && (update_stream == stream || event_a == event_b))
    return set_error(SG_ERR_INVALID_ARGUMENT,
                     "update_stream must differ from stream, and event_a from event_b");
  if (sg_status e = check_device()) return e;
  return launch_prepare_hinv(Hinv, H, n, damp, info, workspace, static_cast<hipStream_t>(stream),
                             static_cast<hipStream_t>(update_stream), static_cast<hipEvent_t>(event_a),
                             static_cast<hipEvent_t>(event_b));
}

sg_status sg_prepare_hinv_batched(float* const* Hinv, const float* const* H, int32_t num_layers, int64_t n,
                                  double damp, int32_t* info, void* workspace, size_t ws_bytes, void* stream,
                                  void* update_stream, void* event_a, void* event_b) {
  g_last_error.clear();
  if (!Hinv || !H || !info) return set_error(SG_ERR_INVALID_ARGUMENT, "Hinv, H and info must not be NULL");
  if (num_layers < 1 || num_layers > SG_MAX_SEGMENTS)
    return set_error(SG_ERR_INVALID_ARGUMENT, "num_layers=%d out of [1, %d]", num_layers, SG_MAX_SEGMENTS);
  if (n < 1 || n > 65536) return set_error(SG_ERR_INVALID_ARGUMENT, "n=%lld out of [1, 65536]", (long long)n);
  if (!(damp >= 0.0) || !isfinite(damp))
    return set_error(SG_ERR_INVALID_ARGUMENT, "damp must be finite and >= 0");
  for (int L = 0; L < num_layers; ++L) {
    if (!Hinv[L] || !H[L]) return set_error(SG_ERR_INVALID_ARGUMENT, "Hinv[%d] and H[%d] must not be NULL", L, L);
    for (int M = 0; M < num_layers; ++M)
      if (static_cast<const void*>(Hinv[L]) == static_cast<const void*>(H[M]))
        return set_error(SG_ERR_INVALID_ARGUMENT, "Hinv[%d] must not alias H[%d]", L, M);
    for (int M = 0; M < L; ++M)
      if (Hinv[L] == Hinv[M]) return set_error(SG_ERR_INVALID_ARGUMENT, "Hinv[%d] and Hinv[%d] are the same", M, L);
  }
  const size_t per = factor_ws_bytes(n);
  if (per > SIZE_MAX / (size_t)num_layers)
    return set_error(SG_ERR_WORKSPACE, "workspace size overflows size_t");
  const size_t need = per * (size_t)num_layers;
  if (!workspace || ws_bytes < need)
    return set_error(SG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned(workspace, 256))
    return set_error(SG_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const int given = (update_stream != nullptr) + (event_a != nullptr) + (event_b != nullptr);
  if (given != 0 && given != 3)
    return set_error(SG_ERR_INVALID_ARGUMENT, "update_stream, event_a and event_b go together (all or none)");
  if (given == 3 && (update_stream == stream || event_a == event_b))
    return set_error(SG_ERR_INVALID_ARGUMENT,
                     "update_stream must differ from stream, and event_a from event_b");
  if (sg_status e = check_device()) return e;
  return launch_prepare_hinv_batched(Hinv, H, num_layers, n, damp, info, workspace,
                                     static_cast<hipStream_t>(stream), static_cast<hipStream_t>(update_stream),
                                     static_cast<hipEvent_t>(event_a), static_cast<hipEvent_t>(event_b));
}

static sg_status prune_common(float* W_out, uint8_t* mask_out, uint8_t* codes_out, float* scale_out,
                              float* zero_out, int32_t bits, const void* W, int32_t w_dtype, int64_t m,
                              int64_t n, int64_t ldw, const int64_t* row_splits, int32_t nseg,
                              const float* Hinv, int32_t pattern_kind,
                              double sparsity, int32_t n_keep, int32_t m_group, int32_t blocksize,
                              const uint8_t* mask_in, void* workspace, size_t ws_bytes, void* stream,
                              int32_t vec = 1, const float* const* Useg = nullptr) {
  if (!W_out || !W || !Hinv) return set_error(SG_ERR_INVALID_ARGUMENT, "W_out, W and Hinv must not be NULL");
  if (m < 1 || n < 1) return set_error(SG_ERR_INVALID_ARGUMENT, "m and n must be >= 1");
  if ((unsigned long long)m * (unsigned long long)n >= (1ull << 32))
    return set_error(SG_ERR_UNSUPPORTED, "m*n must be < 2^32");
  if (ldw < n) return set_error(SG_ERR_INVALID_ARGUMENT, "ldw=%lld < n=%lld", (long long)ldw, (long long)n);
  if (w_dtype != SG_F32 && w_dtype != SG_BF16)
    return set_error(SG_ERR_UNSUPPORTED, "w_dtype %d not supported", w_dtype);
  if (static_cast<const void*>(W_out) == W && !(w_dtype == SG_F32 && ldw == n))
    return set_error(SG_ERR_INVALID_ARGUMENT, "W_out may alias W only for fp32 W with ldw == n");
  if (blocksize < 1 || blocksize > SG_MAX_BLOCKSIZE)
    return set_error(SG_ERR_UNSUPPORTED, "blocksize %d out of [1, %d]", blocksize, SG_MAX_BLOCKSIZE);
  if (pattern_kind == SG_UNSTRUCTURED || pattern_kind == SG_UNSTRUCTURED_ROW) {
    if (!(sparsity >= 0.0 && sparsity <= 1.0))
      return set_error(SG_ERR_INVALID_ARGUMENT, "sparsity must lie in [0, 1]");
  } else if (pattern_kind == SG_NM) {
    if (m_group < 1 || n_keep < 0 || n_keep > m_group)
      return set_error(SG_ERR_INVALID_ARGUMENT, "N:M needs 0 <= N <= M, M >= 1");
    if (n % m_group != 0)
      return set_error(SG_ERR_INVALID_ARGUMENT, "M=%d must divide n=%lld", m_group, (long long)n);
    if (blocksize % m_group != 0)
      return set_error(SG_ERR_INVALID_ARGUMENT, "M=%d must divide blocksize=%d", m_group, blocksize);
    if (!((m_group <= 16 && 16 % m_group == 0) || m_group % 16 == 0))
      return set_error(SG_ERR_UNSUPPORTED, "M=%d: groups must divide 16 or be a multiple of 16", m_group);
  } else {
    return set_error(SG_ERR_INVALID_ARGUMENT, "unknown pattern kind %d", pattern_kind);
  }
  const size_t need = prune_ws_bytes(m, n, blocksize);
  if (!workspace || ws_bytes < need)
    return set_error(SG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned(workspace, 256))
    return set_error(SG_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (sg_status e = check_device()) return e;
  PruneArgs a;
  a.W_out = W_out;
  a.mask_out = mask_out;
  a.W = W;
  a.w_dtype = w_dtype;
  a.m = m;
  a.n = n;
  a.ldw = ldw;
  a.U = Hinv;
  a.seg_u = Useg != nullptr;
  for (int p = 0; p < SG_MAX_SEGMENTS; ++p) a.Useg[p] = (Useg && p < nseg) ? Useg[p] : Hinv;
  a.kind = pattern_kind;
  a.sparsity = sparsity;
  a.n_keep = pattern_kind == SG_NM ? n_keep : 0;
  a.m_group = pattern_kind == SG_NM ? m_group : 1;
  a.blocksize = blocksize;
  a.mask_in = mask_in;
  a.vec = vec;
  a.nseg = nseg;
  a.seg_rows[0] = 0;
  for (int p = 1; p <= nseg; ++p) a.seg_rows[p] = row_splits ? row_splits[p] : m;
  a.bits = bits;
  a.codes_out = codes_out;
  a.qscale = scale_out;
  a.qzero = zero_out;
  return launch_prune(a, workspace, static_cast<hipStream_t>(stream));
}

sg_status sg_prune_layer(float* W_out, uint8_t* mask_out, const void* W, int32_t w_dtype, int64_t m,
                         int64_t n, int64_t ldw, const float* Hinv, int32_t pattern_kind,
                         double sparsity, int32_t n_keep, int32_t m_group, int32_t blocksize,
                         const uint8_t* mask_in, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  return prune_common(W_out, mask_out, nullptr, nullptr, nullptr, 0, W, w_dtype, m, n, ldw, nullptr, 1,
                      Hinv, pattern_kind, sparsity, n_keep, m_group, blocksize, mask_in, workspace,
                      ws_bytes, stream);
}

sg_status sg_prune_layer_noalloc(float* W_out, uint8_t* mask_out, const void* W, int32_t w_dtype,
                                 int64_t m, int64_t n, int64_t ldw, const float* Hinv,
                                 int32_t pattern_kind, double sparsity, int32_t n_keep,
                                 int32_t m_group, int32_t blocksize, const uint8_t* mask_in,
                                 void* stream) {
  g_last_error.clear();
  if (!W_out || !W || !Hinv) return set_error(SG_ERR_INVALID_ARGUMENT, "W_out, W and Hinv must not be NULL");
  if (m < 1 || n < 1) return set_error(SG_ERR_INVALID_ARGUMENT, "m and n must be >= 1");
  if (blocksize < 1 || blocksize > SG_MAX_BLOCKSIZE)
    return set_error(SG_ERR_UNSUPPORTED, "blocksize %d out of [1, %d]", blocksize, SG_MAX_BLOCKSIZE);
  const size_t need = prune_ws_bytes(m, n, blocksize);
  if (need > kNoAllocScratchBytes)
    return set_error(SG_ERR_UNSUPPORTED,
                     "m=%lld needs %zu bytes of scratch; sg_prune_layer_noalloc holds %zu "
                     "(use sg_prune_layer with a workspace)",
                     (long long)m, need, kNoAllocScratchBytes);
  if (sg_status e = check_device()) return e;
  void* ws = nullptr;
  if (sg_status e = noalloc_scratch(&ws)) return e;
  return prune_common(W_out, mask_out, nullptr, nullptr, nullptr, 0, W, w_dtype, m, n, ldw, nullptr, 1,
                      Hinv, pattern_kind, sparsity, n_keep, m_group, blocksize, mask_in, ws,
                      kNoAllocScratchBytes, stream);
}

sg_status sg_prune_quantize_layer(float* W_out, uint8_t* mask_out, uint8_t* codes_out, float* scale_out,
                                  float* zero_out, int32_t bits, const void* W, int32_t w_dtype,
                                  int64_t m, int64_t n, int64_t ldw, const float* Hinv,
                                  int32_t pattern_kind, double sparsity, int32_t n_keep,
                                  int32_t m_group, int32_t blocksize, const uint8_t* mask_in,
                                  void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!scale_out || !zero_out) return set_error(SG_ERR_INVALID_ARGUMENT, "scale_out and zero_out must not be NULL");
  if (bits < 2 || bits > 8) return set_error(SG_ERR_INVALID_ARGUMENT, "bits=%d out of [2, 8]", bits);
  return prune_common(W_out, mask_out, codes_out, scale_out, zero_out, bits, W, w_dtype, m, n, ldw,
                      nullptr, 1, Hinv, pattern_kind, sparsity, n_keep, m_group, blocksize, mask_in,
                      workspace, ws_bytes, stream);
}

sg_status sg_prune_layer_vector(float* W_out, uint8_t* mask_out, const void* W, int32_t w_dtype,
                                int64_t m, int64_t n, int64_t ldw, const float* Hinv,
                                int32_t pattern_kind, double sparsity, int32_t n_keep,
                                int32_t m_group, int32_t blocksize, int32_t vec,
                                const uint8_t* mask_in, void* workspace, size_t ws_bytes,
                                void* stream) {
  g_last_error.clear();
  if (vec != 1 && vec != 16) return set_error(SG_ERR_UNSUPPORTED, "vec=%d: 1 or 16 supported", vec);
  if (vec == 16) {
    if (blocksize % 16 != 0)
      return set_error(SG_ERR_INVALID_ARGUMENT, "vec=16 needs a block size that is a multiple of 16");
    if (pattern_kind == SG_NM && 16 % m_group != 0 && m_group % 16 != 0)
      return set_error(SG_ERR_INVALID_ARGUMENT, "vec=16 needs M | 16 or 16 | M");
  }
  return prune_common(W_out, mask_out, nullptr, nullptr, nullptr, 0, W, w_dtype, m, n, ldw, nullptr, 1,
                      Hinv, pattern_kind, sparsity, n_keep, m_group, blocksize, mask_in, workspace,
                      ws_bytes, stream, vec);
}

sg_status sg_prune_layers_shared(float* W_out, uint8_t* mask_out, uint8_t* codes_out, float* scale_out,
                                 float* zero_out, int32_t bits, const void* W, int32_t w_dtype,
                                 int64_t m_total, int64_t n, int64_t ldw, const int64_t* row_splits,
                                 int32_t nseg, const float* Hinv, int32_t pattern_kind, double sparsity,
                                 int32_t n_keep, int32_t m_group, int32_t blocksize,
                                 const uint8_t* mask_in, void* workspace, size_t ws_bytes,
                                 void* stream) {
  g_last_error.clear();
  if (!row_splits) return set_error(SG_ERR_INVALID_ARGUMENT, "row_splits must not be NULL");
  if (nseg < 1 || nseg > SG_MAX_SEGMENTS)
    return set_error(SG_ERR_INVALID_ARGUMENT, "nseg=%d out of [1, %d]", nseg, SG_MAX_SEGMENTS);
  if (row_splits[0] != 0 || row_splits[nseg] != m_total)
    return set_error(SG_ERR_INVALID_ARGUMENT, "row_splits must run from 0 to m_total");
  for (int p = 0; p < nseg; ++p)
    if (row_splits[p + 1] <= row_splits[p])
      return set_error(SG_ERR_INVALID_ARGUMENT, "row_splits must increase strictly");
  if (bits != 0) {
    if (bits < 2 || bits > 8) return set_error(SG_ERR_INVALID_ARGUMENT, "bits=%d: 0 or [2, 8]", bits);
    if (!scale_out || !zero_out)
      return set_error(SG_ERR_INVALID_ARGUMENT, "scale_out and zero_out must not be NULL when bits > 0");
  }
  return prune_common(W_out, mask_out, bits ? codes_out : nullptr, bits ? scale_out : nullptr,
                      bits ? zero_out : nullptr, bits, W, w_dtype, m_total, n, ldw, row_splits, nseg,
                      Hinv, pattern_kind, sparsity, n_keep, m_group, blocksize, mask_in, workspace,
                      ws_bytes, stream);
}

sg_status sg_prune_layers_batched(float* W_out, uint8_t* mask_out, uint8_t* codes_out, float* scale_out,
                                  float* zero_out, int32_t bits, const void* W, int32_t w_dtype,
                                  int64_t m_total, int64_t n, int64_t ldw, const int64_t* row_splits,
                                  int32_t nseg, const float* const* Hinv, int32_t pattern_kind,
                                  double sparsity, int32_t n_keep, int32_t m_group, int32_t blocksize,
                                  const uint8_t* mask_in, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!row_splits || !Hinv) return set_error(SG_ERR_INVALID_ARGUMENT, "row_splits and Hinv must not be NULL");
  if (nseg < 1 || nseg > SG_MAX_SEGMENTS)
    return set_error(SG_ERR_INVALID_ARGUMENT, "nseg=%d out of [1, %d]", nseg, SG_MAX_SEGMENTS);
  if (row_splits[0] != 0 || row_splits[nseg] != m_total)
    return set_error(SG_ERR_INVALID_ARGUMENT, "row_splits must run from 0 to m_total");
  for (int p = 0; p < nseg; ++p) {
    if (row_splits[p + 1] <= row_splits[p])
      return set_error(SG_ERR_INVALID_ARGUMENT, "row_splits must increase strictly");
    if (!Hinv[p]) return set_error(SG_ERR_INVALID_ARGUMENT, "Hinv[%d] is NULL", p);
  }
  if (bits != 0) {
    if (bits < 2 || bits > 8) return set_error(SG_ERR_INVALID_ARGUMENT, "bits=%d: 0 or [2, 8]", bits);
    if (!scale_out || !zero_out)
      return set_error(SG_ERR_INVALID_ARGUMENT, "scale_out and zero_out must not be NULL when bits > 0");
  }
  return prune_common(W_out, mask_out, bits ? codes_out : nullptr, bits ? scale_out : nullptr,
                      bits ? zero_out : nullptr, bits, W, w_dtype, m_total, n, ldw, row_splits, nseg,
                      Hinv[0], pattern_kind, sparsity, n_keep, m_group, blocksize, mask_in, workspace,
                      ws_bytes, stream, 1, Hinv);
}

sg_status sg_reconstruction_error(double* err, int32_t accumulate, const void* W, int32_t w_dtype,
                                  int64_t ldw, const float* W_hat, int64_t m, int64_t n,
                                  const void* X, int32_t x_dtype, int64_t T, int64_t ldx,
                                  void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!err || !W || !W_hat || !X)
    return set_error(SG_ERR_INVALID_ARGUMENT, "err, W, W_hat and X must not be NULL");
  if (m < 1 || n < 1 || T < 1) return set_error(SG_ERR_INVALID_ARGUMENT, "m, n, T must be >= 1");
  if (ldw < n || ldx < n) return set_error(SG_ERR_INVALID_ARGUMENT, "ldw and ldx must be >= n");
  if ((w_dtype != SG_F32 && w_dtype != SG_BF16) || (x_dtype != SG_F32 && x_dtype != SG_BF16))
    return set_error(SG_ERR_UNSUPPORTED, "dtype not supported");
  if (ceil_div(m, kRecTile) > 65535) return set_error(SG_ERR_UNSUPPORTED, "m too large");
  const size_t need = recon_ws_bytes(m, T);
  if (!workspace || ws_bytes < need)
    return set_error(SG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned(workspace, 256))
    return set_error(SG_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (sg_status e = check_device()) return e;
  return launch_recon(err, accumulate, W, w_dtype, ldw, W_hat, m, n, X, x_dtype, T, ldx, workspace,
                      static_cast<hipStream_t>(stream));
}

sg_status sg_pack_two_four(void* values, int32_t v_dtype, uint8_t* meta, int32_t* bad,
                           const float* W_hat, const uint8_t* mask, int64_t m, int64_t n,
                           void* stream) {
  g_last_error.clear();
  if (!values || !meta || !bad || !W_hat || !mask)
    return set_error(SG_ERR_INVALID_ARGUMENT, "values, meta, bad, W_hat and mask must not be NULL");
  if (m < 1 || n < 4) return set_error(SG_ERR_INVALID_ARGUMENT, "m must be >= 1 and n >= 4");
  if (n % 4 != 0) return set_error(SG_ERR_INVALID_ARGUMENT, "n=%lld is not a multiple of 4", (long long)n);
  if ((unsigned long long)m * (unsigned long long)n >= (1ull << 40))
    return set_error(SG_ERR_UNSUPPORTED, "m*n too large");
  if (v_dtype != SG_F32 && v_dtype != SG_BF16)
    return set_error(SG_ERR_UNSUPPORTED, "v_dtype %d not supported", v_dtype);
  if (sg_status e = check_device()) return e;
  return launch_pack_two_four(values, v_dtype, meta, bad, W_hat, mask, m, n,
                              static_cast<hipStream_t>(stream));
}

}  // extern "C"
