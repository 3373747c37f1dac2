/*
 * flce.h -- fused linear cross-entropy (LM-head projection + token-level
 * cross-entropy, forward and backward) on AMD Instinct MI355X (gfx950).
 *
 * What is computed (one call = one forward + backward pass):
 *
 *   Z  = h . W^T                        logits, never stored in device memory
 *   Z' = s * tanh(Z / s)  if s > 0      softcap ("logit_softcapping", NeMo
 *        Z                otherwise     AutoModel linear_ce page, API)
 *   lse_i = log sum_v exp(Z'_iv)
 *   l_i   = lse_i - Z'_{i,y_i}  if y_i != ignore_index, else 0
 *   loss  = c * sum_i l_i                (accumulated in float64, returned fp32)
 *   G     = c * valid * (softmax(Z') - onehot(y)) * dZ'/dZ
 *   dH    = G . W,   dW = G^T . h
 *
 * with the scale c fixed by the reduction contract:
 *   'sum'  : c = mb_scale / T if num_label_tokens T > 0, else mb_scale
 *            (NeMo AutoModel linear_ce page, API, forward parameter
 *            num_label_tokens: the global count normalises a sum loss)
 *   'mean' : c = mb_scale / max(n, 1), n = number of non-ignored tokens
 *            (the clamped count gives an empty target set loss 0, not NaN:
 *            Ling-3.1-flash discussion 7, "Why use num_items_in_batch")
 * and num_tokens = n for 'sum' and 0 for 'mean' (twinkle PR 335,
 * "PR information", item 1). mb_scale is the token-weighted micro-batch scale
 * (same PR, item 2: 1.0 for 'sum'). The loss is float32 also for bf16 inputs
 * and no logit is ever rounded to bf16 (Modalities PR 464, "The problem" and
 * "Tests"). The softcap is applied identically to the log-sum-exp, the target
 * logit and the gradient (twinkle PR 335, item 3).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps no pointer after a call returns and allocates no device memory.
 *   - Matrices are dense row-major: h [N,H], W [V,H], dH [N,H], dW [V,H];
 *     labels int64 [N]. Batch/sequence dimensions are flattened by the caller;
 *     labels are already aligned row-for-row with h (no internal shift).
 *   - dtype FLCE_BF16: h, W, dH, dW are bfloat16 (dH/dW rounded to nearest
 *     even from float32 accumulators); FLCE_F32: all four are float32.
 *   - stream is a hipStream_t (NULL = the null stream). All work is queued on
 *     it; outputs are valid once the stream reaches that point.
 *   - Return value: an flce_status_t. A non-OK value from the synchronous
 *     argument checks means nothing was launched and nothing was written.
 *   - A call allocates nothing, never waits for the device and clears memory
 *     with kernels (no memset nodes), so it can be captured into a HIP graph
 *     and replayed, with the pointers it was captured with (profiling off).
 *   - Each call opens ROCTX ranges (the entry point's name, then
 *     "flce.setup", "flce.forward", one "flce.backward_chunk" per vocabulary
 *     chunk, ...) around the launches it enqueues, for a profiler's marker
 *     trace; they cost nothing measurable without one.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FLCE_F32 = 0, FLCE_BF16 = 1 } flce_dtype_t;
typedef enum { FLCE_SUM = 0, FLCE_MEAN = 1 } flce_reduction_t;

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_ARG = 1,          /* invalid argument (shape, pointer, option)   */
  FLCE_ERR_UNSUPPORTED = 2,  /* valid but not supported (alignment, shape)  */
  FLCE_ERR_WORKSPACE = 3,    /* workspace missing, misaligned or too small  */
  FLCE_ERR_HIP = 4,          /* a HIP runtime call or launch failed         */
  FLCE_ERR_LABEL = 5,        /* device-detected: a non-ignored label is
                                outside [0, V); reported through *status     */
  FLCE_ERR_SCRATCH = 6       /* the problem needs more scratch than the fixed
                                array of flce_forward_noalloc holds          */
} flce_status_t;

/*
 * flce_workspace_size -- bytes of device scratch that flce_forward_backward
 * needs for this problem (256-byte aligned base required). It holds the
 * per-tile log-sum-exp partials, the per-token lse and target logits, one
 * vocabulary chunk of the logit gradient, (bf16, several chunks) a float32
 * dH accumulator and (bf16, N*H under 128 tiles of 256 x 256) up to 8 float32
 * N x H partial products of a dH split along the vocabulary. Never O(N*V)
 * beyond a fixed fraction: the chunk holds up to 2^27 elements of G, or up to
 * N*V*4/16 bytes when that is more (at most 2^29 elements), and the
 * vocabulary is split into chunks of equal size.
 * Returns 0 for invalid sizes (N < 0, H <= 0, V <= 0, unknown dtype).
 * Pure host arithmetic; callable without a GPU. No page defines this call:
 * it is this library's own addition, so that the caller owns every byte of
 * device memory the step uses.
 */
size_t flce_workspace_size(int64_t N, int64_t H, int64_t V, int dtype);

/*
 * flce_check_args -- the synchronous argument checks of flce_forward_backward,
 * with the same parameter list, without touching the GPU (pointers are only
 * compared, never dereferenced). This library's own addition (no page
 * defines it), so the checks can be tested on a machine without a GPU.
 * Returns FLCE_OK or the error that flce_forward_backward would return
 * before launching anything:
 *   FLCE_ERR_ARG         N < 0, H <= 0, V <= 0; a required pointer is NULL
 *                        (h, W, labels, dH when N > 0; loss, num_tokens, dW
 *                        always); unknown dtype/reduction; softcap < 0 or not
 *                        finite; mb_scale negative or not finite;
 *                        num_label_tokens > 0 with 'mean'; a gradient output
 *                        (dH, dW) overlapping an input matrix (h, W), the other
 *                        gradient, the labels, loss, num_tokens, status,
 *                        lse_out or the workspace.
 *   FLCE_ERR_UNSUPPORTED a bf16 matrix pointer (h, W, dH, dW) not 16-byte
 *                        aligned.
 * Any H > 0 is accepted (the NeMo linear_ce page, "API", puts no limit on the
 * hidden size). The kernels load and store whole 16-byte runs of a bf16 row,
 * so with bf16 inputs and H % 8 != 0 the call runs at the width rounded up to
 * 8 on copies in the workspace: W and the gathered hidden rows zero-padded
 * (a padded copy of h for the entry points that do not gather), dW (from the
 * caller's one when accumulate_dW) and dH computed at that width and copied
 * out to the caller's H columns. The results equal those of the same call on
 * inputs the caller padded with zeros; the workspace grows by the padded
 * copies (the *_workspace_size functions count them).
 *   FLCE_ERR_WORKSPACE   workspace NULL, not 256-byte aligned, or
 *                        workspace_bytes < flce_workspace_size(...).
 */
int flce_check_args(const void* h, const void* W, const int64_t* labels,
                    int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                    float softcap, int reduction, int64_t num_label_tokens,
                    float* loss, int64_t* num_tokens, void* dH, void* dW,
                    void* stream, int dtype, float mb_scale, int accumulate_dW,
                    void* workspace, size_t workspace_bytes, int32_t* status,
                    float* lse_out);

/*
 * flce_forward_backward -- the whole fused linear cross-entropy step.
 *
 * Inputs  h [N,H], W [V,H], labels [N] (int64), ignore_index (compared by
 *         equality; may name a vocabulary row), softcap s >= 0 (0 = off),
 *         reduction (flce_reduction_t), num_label_tokens T (<= 0: absent;
 *         only with 'sum'), dtype (flce_dtype_t), mb_scale (finite and
 *         >= 0: the token-weighted micro-batch scale is a token fraction
 *         n_mb / n_total, 1.0 for a plain call; 0 gives loss 0 and zero
 *         gradients; negative is FLCE_ERR_ARG), accumulate_dW (0: dW is
 *         overwritten, and until the call writes its rows it also holds
 *         intermediate values of the call (the logit gradient of some
 *         vocabulary chunks, which saves recomputing their logits), so its
 *         contents are only defined once the call has completed; 1: the
 *         computed gradient is added to the dW already in memory, for
 *         micro-batching).
 * Outputs *loss (fp32 scalar), *num_tokens (int64 scalar), dH [N,H],
 *         dW [V,H], optional lse_out [N] fp32 (per-token log-sum-exp of the
 *         softcapped logits; NULL = not written), optional *status (int32:
 *         FLCE_OK, or FLCE_ERR_LABEL when a non-ignored label is outside
 *         [0, V); NULL = not written). All are device pointers.
 * Workspace caller-owned device scratch of workspace_bytes >=
 *         flce_workspace_size(N, H, V, dtype); its contents on entry do not
 *         matter and are garbage on exit. Two calls may run concurrently only
 *         with distinct workspaces.
 * Edge cases N = 0: loss 0, num_tokens 0, dW zero-filled unless
 *         accumulate_dW. Every label ignored: loss 0 and zero gradients for
 *         both reductions (no NaN).
 * Data errors (detected on the device, after launch): a non-ignored label
 *         outside [0, V) makes *status = FLCE_ERR_LABEL, *loss = NaN, that
 *         token's dH row NaN and dW NaN (fail closed); nothing is read or
 *         written out of bounds.
 * Errors  see flce_check_args; FLCE_ERR_HIP if a launch fails.
 */
int flce_forward_backward(const void* h, const void* W, const int64_t* labels,
                          int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                          float softcap, int reduction, int64_t num_label_tokens,
                          float* loss, int64_t* num_tokens, void* dH, void* dW,
                          void* stream, int dtype, float mb_scale, int accumulate_dW,
                          void* workspace, size_t workspace_bytes, int32_t* status,
                          float* lse_out);

/*
 * float32 gradients for bf16 inputs (the *_ex entry points): the same call
 * with one more argument, grad_dtype, the dtype of dH and dW. grad_dtype ==
 * dtype is exactly flce_forward_backward. dtype FLCE_BF16 with grad_dtype
 * FLCE_F32 writes dH and dW as float32 (dW added in float32 when
 * accumulate_dW is set), so a caller can accumulate gradients over
 * micro-batches in float32 (twinkle PR 335, "PR information", item 2: the
 * token-weighted micro-batch scale; Modalities PR 464, "What the reference
 * implementations do": the chunked path there accumulates its gradients in
 * float32). The logit gradient G, otherwise rounded to bf16
 * once, is kept as a pair G = G_hi + G_lo of bf16 values (G_hi = bf16(G),
 * G_lo = bf16(G - G_hi)), about 16 significant bits, and each gradient GEMM
 * runs once per part in a fixed order: twice the dW/dH work of the bf16
 * call. dtype FLCE_F32 with grad_dtype FLCE_BF16 is FLCE_ERR_UNSUPPORTED.
 * Float32 gradients need the matrix pointers dH, dW 16-byte aligned like
 * the bf16 ones, and any H is padded the same way. The workspace is
 * flce_workspace_size_ex(N, H, V, dtype, grad_dtype) bytes and
 * flce_vocab_chunk_ex gives the vocabulary chunk (half the bf16 call's).
 */
size_t flce_workspace_size_ex(int64_t N, int64_t H, int64_t V, int dtype, int grad_dtype);
int64_t flce_vocab_chunk_ex(int64_t N, int64_t H, int64_t V, int dtype, int grad_dtype);
int flce_check_args_ex(const void* h, const void* W, const int64_t* labels,
                       int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                       float softcap, int reduction, int64_t num_label_tokens,
                       float* loss, int64_t* num_tokens, void* dH, void* dW,
                       void* stream, int dtype, float mb_scale, int accumulate_dW,
                       void* workspace, size_t workspace_bytes, int32_t* status,
                       float* lse_out, int grad_dtype);
int flce_forward_backward_ex(const void* h, const void* W, const int64_t* labels,
                             int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                             float softcap, int reduction, int64_t num_label_tokens,
                             float* loss, int64_t* num_tokens, void* dH, void* dW,
                             void* stream, int dtype, float mb_scale, int accumulate_dW,
                             void* workspace, size_t workspace_bytes, int32_t* status,
                             float* lse_out, int grad_dtype);

/*
 * The no-recompute variant (bf16 only): the same call and results, with one
 * more argument, token_chunk. Instead of recomputing the logits in the
 * backward pass (2*N*H*V flop), it goes through the tokens in chunks of
 * token_chunk (rounded up to 256; <= 0: min(N, 8192) rounded up) and keeps
 * each chunk's probabilities relative to each vocabulary tile's max,
 * P'[t][v] = exp(z'_tv - M) <= 1, as bf16 in the workspace; after the chunk's
 * log-sum-exp they become G in place (G = c (P' exp(M - lse) - [v = y])
 * dz'/dz, the target element from its float32 logit), then dW and the
 * chunk's dH. With more than one chunk dW is summed over the chunks in a
 * float32 [V,H] accumulator in the workspace and rounded to bf16 once, after
 * the last chunk (with accumulate_dW the bf16 dW already in memory is its
 * starting value). The chunked path that the Modalities PR 464 page
 * describes ("What the reference implementations do": memory is bounded by
 * chunking the sequence, gradients accumulate in float32) is the model; the
 * logits themselves are never rounded to bf16. Cost: 6*N*H*V flop, plus
 * token_chunk * roundup(V, 256) * 2 bytes of workspace
 * (flce_workspace_size_nr), 2 GiB at N >= 8192, V = 131072 with the default;
 * with several chunks the V*H*4-byte dW accumulator; and, when
 * token_chunk * H is under 128 tiles of 256 x 256, up to 8 float32
 * token_chunk x H partial products of a dH split along the vocabulary. A
 * smaller token_chunk trades speed (one more pass over the dW accumulator per
 * chunk) for memory.
 * Errors as flce_check_args, with FLCE_ERR_UNSUPPORTED for float32 inputs;
 * flce_token_chunk_nr gives the chunk used.
 */
size_t flce_workspace_size_nr(int64_t N, int64_t H, int64_t V, int dtype, int64_t token_chunk);
int64_t flce_token_chunk_nr(int64_t N, int64_t H, int64_t V, int dtype, int64_t token_chunk);
int flce_check_args_nr(const void* h, const void* W, const int64_t* labels,
                       int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                       float softcap, int reduction, int64_t num_label_tokens,
                       float* loss, int64_t* num_tokens, void* dH, void* dW,
                       void* stream, int dtype, float mb_scale, int accumulate_dW,
                       void* workspace, size_t workspace_bytes, int32_t* status,
                       float* lse_out, int64_t token_chunk);
int flce_forward_backward_nr(const void* h, const void* W, const int64_t* labels,
                             int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                             float softcap, int reduction, int64_t num_label_tokens,
                             float* loss, int64_t* num_tokens, void* dH, void* dW,
                             void* stream, int dtype, float mb_scale, int accumulate_dW,
                             void* workspace, size_t workspace_bytes, int32_t* status,
                             float* lse_out, int64_t token_chunk);

/*
 * flce_forward_workspace_size -- bytes of device scratch that flce_forward
 * needs (256-byte aligned base required): the per-tile log-sum-exp partials
 * and the per-token lse, target logits and losses, O(N * V / 256 + N)
 * bytes, and for bf16 the gathered tokens (positions, labels and hidden
 * rows, N * H * 2 bytes). Returns 0 for invalid sizes. Pure host arithmetic.
 */
size_t flce_forward_workspace_size(int64_t N, int64_t H, int64_t V, int dtype);

/*
 * flce_forward_check_args -- the synchronous argument checks of
 * flce_forward, with its parameter list, without touching the GPU. The rules
 * are those of flce_check_args minus everything about dH, dW and
 * accumulate_dW; the workspace is checked against
 * flce_forward_workspace_size(...).
 */
int flce_forward_check_args(const void* h, const void* W, const int64_t* labels,
                            int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                            float softcap, int reduction, int64_t num_label_tokens,
                            float* loss, int64_t* num_tokens, void* stream, int dtype,
                            float mb_scale, void* workspace, size_t workspace_bytes,
                            int32_t* status, float* lse_out);

/*
 * flce_forward -- the forward half alone: loss, num_tokens and (optionally)
 * the per-token lse, with no gradients, for evaluation and any caller that
 * needs the loss but not the logits (LlamaFactory error page "cross_entropy
 * and fused_linear_cross_entropy cannot both be enabled", "What it means":
 * the fused path is the one that never materialises logits; NeMo AutoModel
 * linear_ce page, API: forward returns the scalar loss). It runs the same
 * kernels as the forward part of flce_forward_backward on the same inputs,
 * so *loss, *num_tokens, lse_out and *status are bit-identical to what that
 * call returns; it costs one GEMM pass (2*N*H*V flops) instead of four. With
 * bf16 inputs it gathers the non-ignored tokens first, like that call, and
 * with lse_out NULL the GEMM runs over those tokens only (an ignored token
 * adds nothing to the loss); with lse_out it runs over all N.
 *
 * Parameters as in flce_forward_backward, without dH, dW and accumulate_dW.
 * Workspace caller-owned, >= flce_forward_workspace_size(N, H, V, dtype)
 *         bytes, 256-byte aligned; garbage on exit.
 * Edge cases N = 0: loss 0, num_tokens 0. Every label ignored: loss 0.
 * Data errors a non-ignored label outside [0, V) makes *status =
 *         FLCE_ERR_LABEL and *loss = NaN (fail closed).
 * Errors  see flce_forward_check_args; FLCE_ERR_HIP if a launch fails.
 */
int flce_forward(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                 int64_t V, int64_t ignore_index, float softcap, int reduction,
                 int64_t num_label_tokens, float* loss, int64_t* num_tokens, void* stream,
                 int dtype, float mb_scale, void* workspace, size_t workspace_bytes,
                 int32_t* status, float* lse_out);

/*
 * flce_forward_noalloc -- flce_forward without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. (No page defines
 * it; it is flce_forward with the library's own scratch.)
 *
 * Scratch  a fixed device array of FLCE_NOALLOC_SCRATCH_BYTES inside the
 *          library, one copy on every GPU the library runs on (the GPU of
 *          `stream`; the current device for the null stream), held until the
 *          process ends. The first call on a GPU looks up that copy's device
 *          address (a HIP runtime query, no allocation). This entry does not
 *          gather the non-ignored tokens: its scratch is the forward's
 *          per-tile partials (ceil(V/256) * roundup(N, 256) * 8 bytes) and
 *          per-token arrays (about 16 * roundup(N, 256) bytes), and a problem
 *          whose scratch exceeds the array is refused with FLCE_ERR_SCRATCH
 *          before anything is launched. The call allocates nothing: no
 *          hipMalloc, no hipFree, no allocating library routine.
 * Sharing  every call on one GPU uses that GPU's array, which keeps the last
 *          call's contents (the kernels write everything they read back), so
 *          calls that overlap on one GPU (two streams, or two host threads)
 *          race: the caller must serialise them.
 * Shapes   it does not gather the tokens, to keep its scratch small; with
 *          bf16 inputs and H % 8 != 0 the padded copies of h and W it reads
 *          count against the scratch (FLCE_ERR_SCRATCH beyond it).
 * Everything else (parameters, outputs, edge cases, errors) as in
 * flce_forward, whose results it reproduces bit for bit (the gather changes
 * no value, and the loss sums the per-token losses by original position).
 */
#define FLCE_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int flce_forward_noalloc(const void* h, const void* W, const int64_t* labels, int64_t N,
                         int64_t H, int64_t V, int64_t ignore_index, float softcap,
                         int reduction, int64_t num_label_tokens, float* loss,
                         int64_t* num_tokens, void* stream, int dtype, float mb_scale,
                         int32_t* status, float* lse_out);

/*
 * flce_forward_logits_check_args -- the synchronous checks of
 * flce_forward_logits, with its parameter list, without touching the GPU:
 * those of flce_forward_check_args, and then FLCE_ERR_ARG unless
 * logits_dtype is FLCE_F32 or FLCE_BF16, V <= ld_logits <= 2^31, logits is
 * non-NULL when N > 0, (N - 1) * ld_logits + V < 2^60, and the logits buffer
 * ((N - 1) * ld_logits + V
 * elements from `logits`) overlaps none of h, W, labels, loss, num_tokens,
 * status, lse_out and the workspace; FLCE_ERR_UNSUPPORTED if logits is not
 * aligned to its element size.
 */
int flce_forward_logits_check_args(const void* h, const void* W, const int64_t* labels,
                                   int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                                   float softcap, int reduction, int64_t num_label_tokens,
                                   float* loss, int64_t* num_tokens, void* stream, int dtype,
                                   float mb_scale, void* workspace, size_t workspace_bytes,
                                   int32_t* status, float* lse_out, void* logits,
                                   int64_t ld_logits, int logits_dtype);

/*
 * flce_forward_logits -- flce_forward that also hands back the logits, for
 * callers that need them (LlamaFactory error page "cross_entropy and
 * fused_linear_cross_entropy cannot both be enabled", "Source" and
 * "Solutions": the fused loss never forms the logits, so a caller with
 * require_logits set is switched to plain cross-entropy; here they come out
 * of the same forward pass instead, at the cost of writing them once).
 *
 * logits  device, caller-owned output, row-major by token:
 *         logits[t * ld_logits + v] = z'_tv for t < N, v < V, where z' is
 *         h_t . W_v, softcapped as s * tanh(z / s) when softcap > 0 (the
 *         Z' of the definition at the top of this file). These are the
 *         float32 values the loss and lse are formed from, stored as float32
 *         (logits_dtype FLCE_F32) or rounded to nearest even bf16
 *         (FLCE_BF16). Elements v in [V, ld_logits) are not written. Rows are
 *         stored in 16-byte runs when logits and ld_logits keep every run
 *         16-byte aligned, element by element otherwise.
 * Shapes  the logits come out in the tokens' order, so this entry does not
 *         gather the tokens: with bf16 inputs and H % 8 != 0 it reads a padded
 *         copy of h (and of W) in its workspace.
 * Everything else as in flce_forward, with the same workspace
 * (flce_forward_workspace_size): *loss, *num_tokens, lse_out and *status are
 * bit-identical to what flce_forward returns on the same inputs. Cost: the
 * forward GEMM (2*N*H*V flops) plus N*V stored elements.
 * Errors  see flce_forward_logits_check_args; FLCE_ERR_HIP if a launch fails.
 */
int flce_forward_logits(const void* h, const void* W, const int64_t* labels, int64_t N,
                        int64_t H, int64_t V, int64_t ignore_index, float softcap,
                        int reduction, int64_t num_label_tokens, float* loss,
                        int64_t* num_tokens, void* stream, int dtype, float mb_scale,
                        void* workspace, size_t workspace_bytes, int32_t* status,
                        float* lse_out, void* logits, int64_t ld_logits, int logits_dtype);

/* flce_status_string -- a static, human-readable name for a status code
 * (this library's own addition; no page defines status codes). */
const char* flce_status_string(int status);

/*
 * flce_vocab_chunk -- the vocabulary chunk (rows of W per backward chunk) the
 * library uses for this problem; informational (host arithmetic only; this
 * library's own addition).
 */
int64_t flce_vocab_chunk(int64_t N, int64_t H, int64_t V, int dtype);

/*
 * flce_kept_chunks -- how many of flce_forward_backward's vocabulary chunks
 * (from the first) get their logit gradient from probabilities the forward
 * kept, without recomputing their logits: chunk 0 alone, in the workspace,
 * when accumulate_dW is set; otherwise up to four, all but the last in the
 * rows of dW the call has not yet written and the last in the workspace. 0 for float32 inputs (every chunk recomputed), for N <= 0 and for
 * invalid sizes; at most 4. Informational (host arithmetic only; this
 * library's own addition).
 */
int64_t flce_kept_chunks(int64_t N, int64_t H, int64_t V, int dtype, int accumulate_dW);

/*
 * Per-kernel timing (diagnostics for benchmarks; not thread-safe; this
 * library's own addition, no page defines it).
 * flce_profile_begin() clears the record and makes subsequent
 * flce_forward_backward calls bracket every kernel launch with a pair of
 * HIP events on the call's stream. flce_profile_end() stops recording.
 * flce_profile_query(kind, &ms, &launches) waits for the recorded events and
 * returns the summed elapsed milliseconds and launch count of one kernel kind
 * (0 <= kind < flce_profile_kinds()); flce_kernel_kind_name(kind) names it.
 * Events are created on first use and reused; no device memory is allocated.
 */
int flce_profile_begin(void);
int flce_profile_end(void);
int flce_profile_kinds(void);
const char* flce_kernel_kind_name(int kind);
int flce_profile_query(int kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
