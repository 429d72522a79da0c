// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built host-only by test_sanitize_host.py; no
// kernel is launched).  Every call below either fails argument validation or,
// with plausible arguments, stops at the device check (no GPU is needed): the
// argument checks, the workspace arithmetic, the host arrays of row splits
// and factors, and the error-message formatting run instrumented.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sg.h"

static int failures = 0;

static void expect(sg_status got, sg_status want, const char* what) {
  const char* msg = sg_last_error_message();
  if (got != want || (got != SG_OK && (msg == nullptr || msg[0] == '\0'))) {
    fprintf(stderr, "FAIL %s: status %d (want %d), message '%s'\n", what, got, want, msg ? msg : "(null)");
    ++failures;
  }
}

// A device-looking address that is never dereferenced on the host.
static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  if (sg_abi_version() != SG_ABI_VERSION) ++failures;
  for (int s = -1; s < 8; ++s)
    if (sg_status_string(s) == nullptr || strlen(sg_status_string(s)) == 0) ++failures;

  // workspace arithmetic over a range of shapes, including the largest ones
  const int64_t dims[] = {1, 2, 7, 64, 127, 128, 1000, 4096, 11008, 28672, 65536};
  const int bss[] = {0, 1, 32, 128, 129};
  size_t acc = 0;
  for (int op = -1; op <= 4; ++op)
    for (int64_t m : dims)
      for (int64_t n : dims)
        for (int bs : bss) acc += sg_workspace_bytes(op, m, n, 524288, bs);
  if (acc == 0) ++failures;

  float* H = static_cast<float*>(fake(0x10000));
  float* U = static_cast<float*>(fake(0x20000));
  void* W = fake(0x30000);
  float* Wo = static_cast<float*>(fake(0x40000));
  void* ws = fake(0x100000);
  int32_t* info = static_cast<int32_t*>(fake(0x50000));

  // null pointers and bad sizes
  expect(sg_hessian_accumulate(nullptr, 16, W, SG_BF16, 8, 16, nullptr, 0, nullptr), SG_ERR_INVALID_ARGUMENT,
         "hessian null");
  expect(sg_hessian_accumulate(H, 70000, W, SG_BF16, 8, 70000, nullptr, 0, nullptr), SG_ERR_INVALID_ARGUMENT,
         "hessian n");
  expect(sg_hessian_accumulate(H, 16, fake(0x30002), SG_BF16, 8, 16, nullptr, 0, nullptr), SG_ERR_UNSUPPORTED,
         "hessian alignment");
  expect(sg_prepare_hinv(U, H, 64, -1.0, info, ws, 1 << 30, nullptr, nullptr, nullptr, nullptr),
         SG_ERR_INVALID_ARGUMENT, "prepare damp");
  expect(sg_prepare_hinv(U, H, 64, 0.01, info, ws, 1 << 30, fake(1), fake(2), fake(3), nullptr),
         SG_ERR_INVALID_ARGUMENT, "prepare side stream");
  expect(sg_prepare_hinv(U, H, 64, 0.01, info, ws, 16, nullptr, nullptr, nullptr, nullptr), SG_ERR_WORKSPACE,
         "prepare workspace");
  expect(sg_prune_layer(Wo, nullptr, W, SG_F32, 64, 128, 128, U, SG_NM, 0.0, 3, 2, 128, nullptr, ws, 1 << 30,
                        nullptr),
         SG_ERR_INVALID_ARGUMENT, "prune N > M");
  expect(sg_prune_layer(Wo, nullptr, W, SG_F32, 70000, 70000, 70000, U, SG_UNSTRUCTURED, 0.5, 0, 1, 128,
                        nullptr, ws, 1 << 30, nullptr),
         SG_ERR_UNSUPPORTED, "prune m*n");
  expect(sg_prune_layer_noalloc(Wo, nullptr, W, SG_BF16, 30000, 256, 256, U, SG_UNSTRUCTURED, 0.5, 0, 1, 128,
                                nullptr, nullptr),
         SG_ERR_UNSUPPORTED, "noalloc size");
  expect(sg_reconstruction_error(nullptr, 0, W, SG_F32, 4, Wo, 4, 4, W, SG_F32, 4, 4, nullptr, 0, nullptr),
         SG_ERR_INVALID_ARGUMENT, "recon null");
  expect(sg_pack_two_four(W, SG_F32, static_cast<uint8_t*>(fake(0x60000)), info, Wo,
                          static_cast<uint8_t*>(fake(0x70000)), 4, 10, nullptr),
         SG_ERR_INVALID_ARGUMENT, "pack n");

  // host arrays: row splits and factors at every count up to the maximum
  int64_t splits[SG_MAX_SEGMENTS + 1];
  const float* hv[SG_MAX_SEGMENTS];
  for (int nseg = 1; nseg <= SG_MAX_SEGMENTS; ++nseg) {
    for (int p = 0; p <= nseg; ++p) splits[p] = 64 * p;
    for (int p = 0; p < nseg; ++p) hv[p] = U;
    const int64_t m = 64 * nseg;
    // bad last split, then plausible arguments (stop at the device check)
    splits[nseg] = m + 1;
    expect(sg_prune_layers_shared(Wo, nullptr, nullptr, nullptr, nullptr, 0, W, SG_F32, m, 128, 128, splits,
                                  nseg, U, SG_UNSTRUCTURED, 0.5, 0, 1, 128, nullptr, ws, 1 << 30, nullptr),
           SG_ERR_INVALID_ARGUMENT, "shared splits");
    splits[nseg] = m;
    hv[nseg - 1] = nullptr;
    expect(sg_prune_layers_batched(Wo, nullptr, nullptr, nullptr, nullptr, 0, W, SG_F32, m, 128, 128, splits,
                                   nseg, hv, SG_UNSTRUCTURED, 0.5, 0, 1, 128, nullptr, ws, 1 << 30, nullptr),
           SG_ERR_INVALID_ARGUMENT, "batched null factor");
    hv[nseg - 1] = U;
    const sg_status st = sg_prune_layers_batched(Wo, nullptr, nullptr, nullptr, nullptr, 0, W, SG_F32, m, 128,
                                                 128, splits, nseg, hv, SG_NM, 0.0, 2, 4, 128, nullptr, ws,
                                                 1 << 30, nullptr);
    if (st != SG_ERR_HIP && st != SG_ERR_UNSUPPORTED) {
      fprintf(stderr, "FAIL batched without a device: status %d\n", st);
      ++failures;
    }
  }
  expect(sg_prune_layers_batched(Wo, nullptr, nullptr, nullptr, nullptr, 0, W, SG_F32, 64, 128, 128, splits,
                                 SG_MAX_SEGMENTS + 1, hv, SG_UNSTRUCTURED, 0.5, 0, 1, 128, nullptr, ws, 1 << 30,
                                 nullptr),
         SG_ERR_INVALID_ARGUMENT, "batched nseg");

  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("abi host checks passed\n");
  return 0;
}
