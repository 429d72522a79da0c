/*
 * sg.h -- C ABI of the SparseGPT layer solver for AMD Instinct MI355X (gfx950).
 *
 * One linear layer Y = W X (W: m x n, rows = output channels, columns = input
 * channels).  The four calls follow the method's own order:
 *
 *   1. sg_hessian_accumulate    H += Xc^T Xc over calibration chunks
 *   2. sg_prepare_hinv          U = upper Cholesky factor of (H + lambda I)^{-1}
 *   3. sg_prune_layer           column sweep: select mask, zero, compensate
 *   4. sg_reconstruction_error  ||W X - W_hat X||_F^2 (validation)
 *
 * Sources, cited by page title and section:
 *   [SGR] "SparseGPT: Massive Language Models Can Be Accurately Pruned in
 *         One-Shot" -- review on devpress.csdn.net (sections 6, 7, 8, 11, 14.4)
 *   [SFT] "Sparse Fine-tuning for Inference Acceleration of LLMs" -- review on
 *         tqpw.cn (section 8.4: N:M groups)
 *   [G24] "LLM 2:4 structured sparsity production guide" -- oh-bug.com (2:4
 *         core mechanism: zeros along the reduction axis)
 * The pages do not give damping, the Cholesky route to the inverse, the
 * saliency formula or lazy batching; the readings adopted are stated below.
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory:  every array argument is DEVICE memory owned by the caller, except
 *          the strings returned by sg_status_string / sg_last_error_message.
 *          The library never allocates or frees device memory: scratch space
 *          comes from the caller's `workspace` (size from sg_workspace_bytes,
 *          alignment 256 bytes).  Matrices are row-major with the stated
 *          leading dimension (in elements).
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Every call
 *          only enqueues work on it (and, for sg_prepare_hinv, on a second
 *          stream the caller may pass) and returns; results are valid once
 *          `stream` is synchronised.  No call synchronises the device, and the
 *          library creates no stream or event.
 * Errors:  host-detectable problems (null pointers, bad sizes or patterns,
 *          small workspace, unsupported dtype or alignment, a device that is
 *          not gfx950) return a non-zero sg_status BEFORE anything is
 *          enqueued; sg_last_error_message() then holds a thread-local
 *          explanation.  A failed launch returns SG_ERR_HIP.
 * Threads: the library keeps no state across calls beyond the thread-local
 *          message and a per-device memo of the architecture check (both
 *          guarded), plus the scratch array of sg_prune_layer_noalloc.  Calls
 *          on different streams with disjoint buffers (and, for
 *          sg_prepare_hinv, distinct update streams and events) may run
 *          concurrently.
 * Dtypes:  SG_F32 = IEEE binary32, SG_BF16 = bfloat16 (upper 16 bits of a
 *          binary32), both read and widened exactly to fp32.
 */
#ifndef SG_H_
#define SG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SG_ABI_VERSION 2

typedef int32_t sg_status;

enum {
  SG_OK = 0,
  SG_ERR_INVALID_ARGUMENT = 1,
  SG_ERR_UNSUPPORTED = 2,
  SG_ERR_WORKSPACE = 3,
  SG_ERR_HIP = 4
};

/* element types */
enum { SG_F32 = 0, SG_BF16 = 1 };

/* sparsity pattern kinds */
enum { SG_UNSTRUCTURED = 0, SG_NM = 1, SG_UNSTRUCTURED_ROW = 2 };

/* operations, for sg_workspace_bytes */
enum {
  SG_OP_HESSIAN = 0,
  SG_OP_PREPARE_HINV = 1,
  SG_OP_PRUNE = 2,
  SG_OP_RECON = 3
};

/* Largest supported column block of sg_prune_layer. */
#define SG_MAX_BLOCKSIZE 128

/* Most matrices one sg_prune_layers_shared call can stack. */
#define SG_MAX_SEGMENTS 16

/* Bytes of the device scratch array that sg_prune_layer_noalloc uses in place
 * of a workspace (64 MiB: sg_prune_layer's workspace for m up to 21,600). */
#define SG_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * sg_hessian_accumulate -- H += Xc^T Xc.
 *
 * [SGR] section 7 (the Hessian proxy H = X X^T of the layer inputs) and
 * section 10 (calibration samples serve to estimate H).  Reading: a raw sum
 * over tokens, no 1/N normalisation; call once per chunk of tokens.
 *
 *   H      [n x n] fp32, leading dimension n, in/out.  Must hold a symmetric
 *          matrix on entry (zero it once before the first chunk); on return
 *          it is again fully symmetric (both triangles written).
 *   n      number of input channels, 1 <= n <= 65536.
 *   X      token-major chunk Xc[t, c] (t < T, c < n) with leading dimension
 *          ldx >= n; x_dtype SG_BF16 or SG_F32.  For SG_BF16 the pointer must
 *          be 16-byte aligned and ldx a multiple of 8 below 2^28 (one copy
 *          instruction spans up to four rows with 32-bit offsets); rows are read in
 *          16-byte pieces up to n rounded up to a multiple of 8, so the buffer
 *          must hold (T - 1) * ldx + round_up(n, 8) elements (a [T, ldx]
 *          tensor or a column view of one does); the values in the padding
 *          columns do not affect H.
 *   T      tokens in the chunk, T >= 1.
 *   workspace / ws_bytes: scratch for the token-split partial tiles or,
 *          without a split, for the progress counters that keep the
 *          workgroups of one XCD on the same tokens (they order nothing the
 *          result depends on); the size from
 *          sg_workspace_bytes(SG_OP_HESSIAN, 0, n, T, 0) gives the intended
 *          split.  A smaller workspace (even 0 bytes) is accepted: the call
 *          then splits the tokens less or runs without the counters (results
 *          stay deterministic for a given workspace size).
 * Accumulation is fp32 (bf16 x bf16 products are exact in fp32).  The result
 * is bitwise reproducible for the same inputs and workspace size.
 */
sg_status sg_hessian_accumulate(float* H, int64_t n, const void* X,
                                int32_t x_dtype, int64_t T, int64_t ldx,
                                void* workspace, size_t ws_bytes, void* stream);

/*
 * sg_prepare_hinv -- Hinv = U, the upper-triangular Cholesky factor of
 * (H + lambda I)^{-1}, lambda = damp * mean(diag H).
 *
 * [SGR] section 8: the error of removing a weight and the compensation of the
 * others come from the inverse Hessian.  The pages name no damping and no
 * factor; reading: dampen by a fraction of the mean diagonal, then
 * U^T U = (H + lambda I)^{-1} with U upper triangular, positive diagonal.
 * Row j of U then holds the inverse Hessian of the columns j..n-1 that are
 * still free when column j is processed (U_jj U[j, j:] = first row of
 * ((H + lambda I)[j:, j:])^{-1}).
 * Computed in fp32 as L = chol(J H_d J), U = J L^{-1} J (J reverses indices),
 * with a blocked factorisation whose trailing updates run on MFMA.
 *
 *   Hinv   [n x n] fp32 out, leading dimension n: upper triangle = U, strictly
 *          lower triangle = 0.
 *   H      [n x n] fp32 in (symmetric, e.g. from sg_hessian_accumulate); not
 *          modified.  Hinv must not alias H.
 *   damp   fraction of mean(diag H) added to the diagonal, finite, >= 0.
 *   info   one device int32, written by the call: 0 = success; j+1 = the
 *          factorisation broke down (non-positive or non-finite pivot) at
 *          original column j; n+1 = mean(diag H) is not finite and positive
 *          (e.g. H is zero).  When info != 0 the contents of Hinv are
 *          unspecified.
 *   workspace: sg_workspace_bytes(SG_OP_PREPARE_HINV, 0, n, 0, 0) bytes
 *          (two n_pad x n_pad fp32 matrices, n_pad = n rounded up to 128).
 *   update_stream, event_a, event_b: optional (all NULL, or all three given):
 *          a second hipStream_t on the same device, different from `stream`,
 *          and two distinct hipEvent_t the caller created and owns.  Above
 *          n = 4096 the trailing updates then run on update_stream beside the
 *          panel chain on `stream`, ordered by the two events, and `stream`
 *          waits for update_stream before the call's last kernel; with NULL
 *          every kernel runs on `stream` (same result, bit for bit; slower at
 *          large n).  Up to n = 4096 the three are not used.  Concurrent calls
 *          must not share an update stream or an event.
 */
sg_status sg_prepare_hinv(float* Hinv, const float* H, int64_t n, double damp,
                          int32_t* info, void* workspace, size_t ws_bytes,
                          void* stream, void* update_stream, void* event_a,
                          void* event_b);

/*
 * sg_prepare_hinv_batched -- sg_prepare_hinv for several matrices of the same
 * order n (the Hessians of layers pruned side by side), factored together.
 *
 * "Vector-Based SparseGPT" (voc.com.cn), part 02: the dense inputs of each
 * layer are recorded, so that several layers can be pruned in parallel.  Each
 * matrix goes through exactly the computation of sg_prepare_hinv (the same
 * result, bit for bit); the calls share their launches, so that the
 * latency-bound panel steps of one matrix run on the CUs the others leave
 * idle.
 *
 *   Hinv, H    HOST arrays of num_layers DEVICE pointers, each as in
 *              sg_prepare_hinv ([n x n] fp32, leading dimension n).  No Hinv[L]
 *              may alias any H[M] or another Hinv[M].
 *   num_layers 1 <= num_layers <= SG_MAX_SEGMENTS.
 *   info       DEVICE array of num_layers int32: info[L] is layer L's status,
 *              with the meanings of sg_prepare_hinv.
 *   workspace  num_layers * sg_workspace_bytes(SG_OP_PREPARE_HINV, 0, n, 0, 0)
 *              bytes, 256-byte aligned (layer L uses the L-th equal part).
 *   stream, update_stream, event_a, event_b: as in sg_prepare_hinv (one
 *              update stream serves all layers).
 * Errors as sg_prepare_hinv, plus SG_ERR_INVALID_ARGUMENT for num_layers out
 * of range or aliased outputs.
 */
sg_status sg_prepare_hinv_batched(float* const* Hinv, const float* const* H,
                                  int32_t num_layers, int64_t n, double damp,
                                  int32_t* info, void* workspace, size_t ws_bytes,
                                  void* stream, void* update_stream,
                                  void* event_a, void* event_b);

/*
 * sg_prune_layer -- sparse W_hat with W_hat X ~ W X.
 *
 * [SGR] section 8 (OBS: choose a weight, estimate its error from the inverse
 * Hessian, set it to zero, update the other not-yet-pruned weights of the same
 * row) and section 11 steps 4-5 (columns processed in blocks; prune the given
 * fraction and update the rest); [SFT] section 8.4 and [G24] (N:M keeps N of
 * every M consecutive input columns).  Readings where the pages are silent:
 *   - saliency of weight (r, c) at its selection point: W_hat[r,c]^2 / U_cc^2;
 *   - compensation reaches only columns to the right of the pruned one;
 *   - SG_UNSTRUCTURED: at the start of each column block of width w (the last
 *     block may be narrower) exactly floor(sparsity * m * w) weights of the
 *     whole m x w block are pruned: the smallest keys (saliency, r*n + c),
 *     lower index first on equal saliency;
 *   - SG_UNSTRUCTURED_ROW: at the start of each column block of width w,
 *     every row prunes floor(sparsity * w) of its own w weights, the smallest
 *     keys (saliency, c) of the row (the per-row reading of the same
 *     fraction-per-block rule);
 *   - SG_NM: at each group start (column = 0 mod m_group), per row, the
 *     m_group - n_keep smallest keys (saliency, c) of the group are pruned;
 *   - the compensation of each block reaches the columns after it through one
 *     batched product W[:, i2:] -= Err * U[i1:i2, i2:] (lazy batching, the
 *     same values as the unbatched procedure up to rounding);
 *   - a pruned weight is stored as +0.0.
 *
 *   W_out    [m x n] fp32 out, contiguous (leading dimension n).  May alias W
 *            only if w_dtype == SG_F32 and ldw == n.
 *   mask_out [m x n] uint8 out, contiguous: 1 = pruned (W_out is then +0.0),
 *            0 = kept.  May be NULL.
 *   W        [m x ldw] in, SG_F32 or SG_BF16, not modified (unless aliased).
 *   Hinv     [n x n] fp32 in: the factor from sg_prepare_hinv for this n.
 *   pattern_kind SG_UNSTRUCTURED or SG_UNSTRUCTURED_ROW (use sparsity in
 *            [0, 1]) or SG_NM (uses n_keep, m_group with 0 <= n_keep <=
 *            m_group, m_group dividing both n and blocksize, and either
 *            dividing 16 or a multiple of 16).
 *   blocksize 1 <= blocksize <= SG_MAX_BLOCKSIZE.
 *   mask_in  optional [m x n] uint8 (contiguous, 1 = prune): when not NULL it
 *            replaces the selection (the pattern is still validated).
 *   workspace: sg_workspace_bytes(SG_OP_PRUNE, m, n, 0, blocksize) bytes.
 * Limits: m * n < 2^32 (linear indices are 32-bit tie-break keys).
 */
sg_status sg_prune_layer(float* W_out, uint8_t* mask_out, const void* W,
                         int32_t w_dtype, int64_t m, int64_t n, int64_t ldw,
                         const float* Hinv, int32_t pattern_kind,
                         double sparsity, int32_t n_keep, int32_t m_group,
                         int32_t blocksize, const uint8_t* mask_in,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * sg_prune_layer_noalloc -- sg_prune_layer without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments (minus workspace / ws_bytes), same results bit for bit and
 * same error behaviour as sg_prune_layer.  The scratch comes from a device
 * array of the library of SG_NOALLOC_SCRATCH_BYTES, one per GPU, held from
 * the first call on that GPU until the process ends; the call itself
 * allocates nothing (no hipMalloc, no allocating library routine).
 * Limit: sg_workspace_bytes(SG_OP_PRUNE, m, n, 0, blocksize) must not exceed
 * SG_NOALLOC_SCRATCH_BYTES (m <= 21,600 at any n), else SG_ERR_UNSUPPORTED
 * before anything is enqueued.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (from different streams or threads) race and must be ordered by
 * the caller.  Each call clears what it needs cleared itself, by kernels on
 * `stream` (no memset), so consecutive calls need no reset in between.
 */
sg_status sg_prune_layer_noalloc(float* W_out, uint8_t* mask_out,
                                 const void* W, int32_t w_dtype, int64_t m,
                                 int64_t n, int64_t ldw, const float* Hinv,
                                 int32_t pattern_kind, double sparsity,
                                 int32_t n_keep, int32_t m_group,
                                 int32_t blocksize, const uint8_t* mask_in,
                                 void* stream);

/*
 * sg_prune_quantize_layer -- sg_prune_layer with the kept weights also
 * rounded to a per-row grid of 2^bits levels inside the same column sweep.
 *
 * [SGR] section 15 (a pruned layer's remaining weights can also be quantized
 * to 4 or 8 bits) and section 17 (GPTQ quantizes weights one at a time and
 * compensates each rounding error through the inverse Hessian, the step
 * SparseGPT applies to pruning).  Readings where the pages are silent:
 *   - each row's grid spans its original weights and 0: lo = min(0, min w),
 *     hi = max(0, max w), scale = (hi - lo) / (2^bits - 1) (1 for an all-zero
 *     row), zero point z = round(-lo / scale);
 *   - selection is exactly that of sg_prune_layer (same saliencies, taken on
 *     the current weights); at column j a kept weight x becomes
 *     scale * (clamp(round(x / scale) + z, 0, 2^bits - 1) - z), rounding half
 *     to even, and its error (x - that) / U_jj is compensated on the row's
 *     later columns exactly like the error of a pruned weight.
 *
 *   codes_out [m x n] uint8 out, contiguous, may be NULL: the grid index of
 *             every weight (W_out = scale * (code - zero)); a pruned weight
 *             holds the row's zero point.
 *   scale_out, zero_out [m] fp32 out (not NULL): each row's grid.
 *   bits      2 <= bits <= 8.
 * Every other argument, the workspace and the error behaviour are those of
 * sg_prune_layer.
 */
sg_status sg_prune_quantize_layer(float* W_out, uint8_t* mask_out,
                                  uint8_t* codes_out, float* scale_out,
                                  float* zero_out, int32_t bits, const void* W,
                                  int32_t w_dtype, int64_t m, int64_t n,
                                  int64_t ldw, const float* Hinv,
                                  int32_t pattern_kind, double sparsity,
                                  int32_t n_keep, int32_t m_group,
                                  int32_t blocksize, const uint8_t* mask_in,
                                  void* workspace, size_t ws_bytes,
                                  void* stream);

/*
 * sg_prune_layer_vector -- sg_prune_layer with the chosen weights of each
 * range of vec consecutive columns removed together (vector-level joint
 * compensation).
 *
 * [VSG] parts 01-02: rather than removing weights one after another with a
 * compensation after each, the weights chosen within a range are set to
 * zero together and the kept weights are adjusted jointly.  Readings where
 * the article is silent:
 *   - ranges are [j0, j0 + vec); vec = 1 is exactly sg_prune_layer, vec = 16
 *     removes each row's chosen weights of a 16-column range at once;
 *   - selection rules, counts and saliencies are those of sg_prune_layer; a
 *     selection point inside a range sees the values at the range start;
 *   - at a range start, a row with chosen set P takes the exact multi-weight
 *     OBS update over the free columns F = [j0, n): delta_F =
 *     -w_P (G_PP)^-1 G_P,F with G = (H_d[F,F])^-1 = U_FF^T U_FF; the chosen
 *     weights become +0.0, earlier columns stay as they are.
 *
 *   vec       1 or 16; with 16 the block size must be a multiple of 16 and,
 *             under N:M, M must divide 16 or be a multiple of it.
 * Every other argument, the workspace and the error behaviour are those of
 * sg_prune_layer.
 */
sg_status sg_prune_layer_vector(float* W_out, uint8_t* mask_out, const void* W,
                                int32_t w_dtype, int64_t m, int64_t n,
                                int64_t ldw, const float* Hinv,
                                int32_t pattern_kind, double sparsity,
                                int32_t n_keep, int32_t m_group,
                                int32_t blocksize, int32_t vec,
                                const uint8_t* mask_in, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * sg_prune_layers_shared -- prune several weight matrices that read the same
 * input (the query/key/value projections, or gate and up) in one call with
 * their one shared factor Hinv.
 *
 * [SGR] section 7: H depends only on a layer's inputs, so matrices fed by the
 * same activations share H and U.  The result for each matrix is exactly
 * that of its own sg_prune_layer (or sg_prune_quantize_layer) call; the
 * matrices are only processed together, so that every launch covers all of
 * their rows.
 *
 *   W, W_out, mask_out, mask_in, codes_out: the nseg matrices stacked by
 *             rows (each n columns wide) into one m_total x n matrix, in the
 *             layouts of sg_prune_layer.
 *   row_splits host array of nseg + 1 row offsets: 0 = row_splits[0] <
 *             row_splits[1] < ... < row_splits[nseg] = m_total; matrix p is
 *             rows [row_splits[p], row_splits[p+1]).
 *   nseg      1 <= nseg <= SG_MAX_SEGMENTS.
 *   bits      0 for pruning only (codes_out, scale_out and zero_out unused),
 *             or 2..8 for the joint sweep of sg_prune_quantize_layer
 *             (scale_out and zero_out [m_total] then required).
 *   Unstructured selection counts floor(sparsity * m_p * w) per block of
 *   each matrix p; every other pattern decides row by row.
 * Workspace: sg_workspace_bytes(SG_OP_PRUNE, m_total, n, 0, blocksize).
 */
sg_status sg_prune_layers_shared(float* W_out, uint8_t* mask_out,
                                 uint8_t* codes_out, float* scale_out,
                                 float* zero_out, int32_t bits, const void* W,
                                 int32_t w_dtype, int64_t m_total, int64_t n,
                                 int64_t ldw, const int64_t* row_splits,
                                 int32_t nseg, const float* Hinv,
                                 int32_t pattern_kind, double sparsity,
                                 int32_t n_keep, int32_t m_group,
                                 int32_t blocksize, const uint8_t* mask_in,
                                 void* workspace, size_t ws_bytes,
                                 void* stream);

/*
 * sg_prune_layers_batched -- prune several layers' weight matrices, each with
 * the factor of its own inputs, in one call.
 *
 * [VSG] part 02 (inter-layer parallel sparsity): with every layer's dense
 * inputs recorded beforehand, the layers' solves no longer depend on one
 * another and can be pruned in parallel.  Each matrix's result is exactly
 * that of its own sg_prune_layer (or sg_prune_quantize_layer) call with its
 * own Hinv; the matrices are only processed together, so that every launch
 * of the latency-bound column sweep covers the rows of all of them.
 *
 *   W, W_out, mask_out, mask_in, codes_out, row_splits, nseg, bits,
 *   scale_out, zero_out: as in sg_prune_layers_shared (the matrices stacked
 *             by rows, each n columns wide).
 *   Hinv      host array of nseg device pointers: Hinv[p] is the [n x n]
 *             factor from sg_prepare_hinv of matrix p's inputs.
 *   Selection counts, patterns, workspace and errors as in
 *   sg_prune_layers_shared (unstructured counts per matrix and block).
 */
sg_status sg_prune_layers_batched(float* W_out, uint8_t* mask_out,
                                  uint8_t* codes_out, float* scale_out,
                                  float* zero_out, int32_t bits, const void* W,
                                  int32_t w_dtype, int64_t m_total, int64_t n,
                                  int64_t ldw, const int64_t* row_splits,
                                  int32_t nseg, const float* const* Hinv,
                                  int32_t pattern_kind, double sparsity,
                                  int32_t n_keep, int32_t m_group,
                                  int32_t blocksize, const uint8_t* mask_in,
                                  void* workspace, size_t ws_bytes,
                                  void* stream);

/*
 * sg_reconstruction_error -- *err = (accumulate ? *err : 0)
 *                                   + ||(W - W_hat) Xc^T||_F^2.
 *
 * [SGR] section 6: the layer objective keeps W_hat X as close as possible to
 * W X.  Call per calibration chunk with accumulate = 1 after the first.
 *
 *   err      one device double, in/out.
 *   W        [m x ldw] original weights (SG_F32 or SG_BF16).
 *   W_hat    [m x n] fp32 contiguous (e.g. W_out of sg_prune_layer).
 *   X        token-major chunk [T x ldx] (SG_F32 or SG_BF16, ldx >= n).
 *   workspace: sg_workspace_bytes(SG_OP_RECON, m, n, T, 0) bytes.
 * Products run in fp32 on MFMA; the final sum is fp64 in a fixed order.
 */
sg_status sg_reconstruction_error(double* err, int32_t accumulate,
                                  const void* W, int32_t w_dtype, int64_t ldw,
                                  const float* W_hat, int64_t m, int64_t n,
                                  const void* X, int32_t x_dtype, int64_t T,
                                  int64_t ldx, void* workspace,
                                  size_t ws_bytes, void* stream);

/*
 * sg_pack_two_four -- the 2:4 compressed form of a pruned matrix: its kept
 * values and a 2-bit position for each.
 *
 * [G24] 2:4 core-mechanism section: two of every four consecutive values
 * along the reduction axis are kept, and 2-bit metadata records where they
 * sit.  The page fixes no byte layout; this one is:
 *   - group g of row r is columns 4g .. 4g+3; its two slots hold two distinct
 *     positions i0 < i1: the kept positions, and if fewer than two are kept,
 *     the lowest pruned positions (stored value +0.0);
 *   - values[r * (n/2) + 2g + s] = W_hat at slot s, in v_dtype (SG_F32: the
 *     fp32 value; SG_BF16: rounded to nearest, ties to even);
 *   - meta[r * ceil(n/8) + g/2] holds the nibble i0 | (i1 << 2) of group g,
 *     in the low half of the byte for even g and the high half for odd g;
 *   - a group with more than two kept positions cannot be represented: its
 *     two lowest kept positions are stored and it is counted in *bad.
 *
 *   values  [m x n/2] out, v_dtype, contiguous.
 *   meta    [m x ceil(n/8)] uint8 out, contiguous.
 *   bad     one device int32 out: the number of unrepresentable groups (0
 *           for every mask sg_prune_layer returns with pattern 2:4).
 *   W_hat   [m x n] fp32 in, contiguous (e.g. W_out of sg_prune_layer).
 *   mask    [m x n] uint8 in, contiguous, 1 = pruned.
 *   n       a multiple of 4; m >= 1.
 * Entries of W_hat at pruned positions are not read.
 */
sg_status sg_pack_two_four(void* values, int32_t v_dtype, uint8_t* meta,
                           int32_t* bad, const float* W_hat,
                           const uint8_t* mask, int64_t m, int64_t n,
                           void* stream);

/* Workspace bytes for an operation (m, n, T, blocksize as in its call; pass 0
 * for arguments the operation does not take).  Pure host arithmetic: touches
 * no device.  Returns 0 for invalid arguments. */
size_t sg_workspace_bytes(int32_t op, int64_t m, int64_t n, int64_t T,
                          int32_t blocksize);

/* Static description of a status code. */
const char* sg_status_string(sg_status s);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* sg_last_error_message(void);

/* SG_ABI_VERSION of the loaded library. */
int32_t sg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SG_H_ */
