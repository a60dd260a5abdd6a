/*
 * lnr.h -- C ABI of liblnr: fused attention-softmax and LayerNorm row reductions for
 * AMD Instinct MI355X (gfx950, CDNA4), hand-written HIP kernels.
 *
 * The operations are the reduce kernels of a Transformer layer as the LightSeq line of work
 * describes them:
 *   - "CMU 11-868 L10: Accelerating Transformers on GPUs, and Where LightSeq Finds the Time",
 *     sections "Technique 1: kernel fusion" (LayerNorm and softmax become custom reduce
 *     kernels) and "Technique 2: rewrite the formula, drop a synchronization" (one fused
 *     pass for mu(x) and mu(x^2); the LayerNorm backward as two sums computed together;
 *     softmax as a max then a sum of exponentials; FP32 compute with FP16 storage).
 *   - "CMU 11-868 HW4: Softmax and LayerNorm as fused CUDA kernels", section "Problem
 *     structure and scoring" (masked softmax forward and backward, LayerNorm forward with
 *     eps inside the square root, LayerNorm input gradient and gamma/beta gradients summed
 *     across rows, row-length templates up to 2048) and section "Faster than what?"
 *     (the mask is added to the scores: softmax(inp + mask)).
 *
 * Conventions shared by every entry point
 *   - Storage dtype is LNR_F32 (IEEE binary32) or LNR_F16 (IEEE binary16); all arithmetic
 *     is binary32. fp16 results are rounded to nearest even.
 *   - Tensors are dense, row-major, C-contiguous device buffers (hipMalloc'd or any
 *     device-accessible memory). The caller owns every buffer; the library allocates and
 *     frees nothing and keeps no state between calls, so calls are re-entrant. Two
 *     exceptions, each described at its declaration: layernorm_bw_noalloc's fixed device
 *     array (one per GPU, shared by its calls) and lnr_time_next_launch's per-thread request.
 *   - `stream` is a hipStream_t passed as void* (NULL means the default stream). Every call
 *     only enqueues work on that stream and returns; nothing synchronises.
 *   - Every argument is checked before anything is enqueued. A failed check returns a
 *     nonzero lnr_status and enqueues nothing. A launch the HIP runtime rejects returns
 *     LNR_ERR_HIP. Faults inside a kernel surface at the caller's next synchronisation.
 *     No C++ exception crosses this interface.
 *   - Results are bitwise reproducible: no floating-point atomics; every reduction has a
 *     fixed order that depends only on the shape.
 *   - Sizes of zero are legal and enqueue nothing, except the normalisation backwards
 *     (layernorm_bw, rmsnorm_bw, bdr_layernorm_bw), which still write zero parameter
 *     gradients when N == 0.
 *   - Any tensor may start at any address aligned to its element size (each workspace
 *     states its own alignment). Rows whose byte length is a multiple of 16 and buffers
 *     aligned to 16 bytes take the 128-bit vector kernels; anything else takes a slower
 *     element-wise kernel with identical results up to rounding order.
 */
#ifndef LNR_H
#define LNR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point below is exported from liblnr.so; nothing else is. */
#define LNR_API __attribute__((visibility("default")))

typedef enum { LNR_F32 = 0, LNR_F16 = 1 } lnr_dtype;

typedef enum {
    LNR_OK = 0,
    LNR_ERR_NULL = 1,        /* a required pointer is NULL */
    LNR_ERR_SHAPE = 2,       /* a size is negative / zero where it may not be, or causal with Tq != Tk */
    LNR_ERR_UNSUPPORTED = 3, /* row length beyond LNR_SOFTMAX_MAX_TK or LNR_LAYERNORM_MAX_C */
    LNR_ERR_DTYPE = 4,       /* dtype is not an lnr_dtype value */
    LNR_ERR_ALIGN = 5,       /* a pointer below its element size's alignment, or a workspace below its stated one */
    LNR_ERR_ALIAS = 6,       /* buffers overlap in a way the operation forbids */
    LNR_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than the matching *_workspace_bytes() */
    LNR_ERR_HIP = 8,         /* the HIP runtime rejected a launch */
    LNR_ERR_SCRATCH = 9      /* the shape needs more than the library's fixed scratch array */
} lnr_status;

#define LNR_SOFTMAX_MAX_TK 2048  /* longest row in the HW4 page's row-length template list */
#define LNR_LAYERNORM_MAX_C 8192

/*
 * attn_softmax_fw -- masked, optionally causal softmax over the last axis of attention scores.
 * [HW4 "Problem structure and scoring": future tokens set to -inf, the attention mask added,
 *  a row max, then exponentials summed and normalised; L10 "Technique 2": two reductions.]
 *
 *   For every row r = (b, h, i) of inp [B, H, Tq, Tk]:
 *     z_j = inp[b,h,i,j] + mask[b,j]            (mask term omitted when mask == NULL)
 *     z_j = -inf                 if causal and j > i
 *     out[b,h,i,j] = exp(z_j - max_k z_k) / sum_k exp(z_k - max_k z_k)
 *   A row whose every z_j is -inf is written as all zeros. Positions with z_j = -inf are
 *   written as exact zeros.
 *
 *   out   [B, H, Tq, Tk] dtype, written. May equal inp (in place); no other overlap allowed.
 *   inp   [B, H, Tq, Tk] dtype, read.
 *   mask  [B, Tk] dtype, additive, broadcast over H and Tq (key padding: 0 keeps a key,
 *         -inf removes it), or NULL.
 *   causal nonzero applies the future-token mask and requires Tq == Tk (LNR_ERR_SHAPE).
 *   Limits: 1 <= Tk <= LNR_SOFTMAX_MAX_TK (else LNR_ERR_UNSUPPORTED / LNR_ERR_SHAPE);
 *           B, H, Tq >= 0.
 */
LNR_API int attn_softmax_fw(void *out, const void *inp, const void *mask, int64_t B, int64_t H,
                    int64_t Tq, int64_t Tk, int causal, lnr_dtype dtype, void *stream);

/*
 * attn_softmax_bw -- gradient of attn_softmax_fw with respect to its input scores.
 * [HW4 "Problem structure and scoring": the softmax backward kernel, templated on row length.]
 *
 *   For every row with forward output y = out_fw and upstream gradient dy = dout:
 *     t = sum_j y_j * dy_j ;   dinp_j = y_j * (dy_j - t)
 *   Masked and future positions need no mask argument: y_j = 0 there, so dinp_j = 0.
 *
 *   dinp   [B, H, Tq, Tk] dtype, written. May equal dout (in place); no other overlap.
 *   dout   [B, H, Tq, Tk] dtype, read.
 *   out_fw [B, H, Tq, Tk] dtype, read (the forward output y).
 *   Limits as attn_softmax_fw.
 */
LNR_API int attn_softmax_bw(void *dinp, const void *dout, const void *out_fw, int64_t B, int64_t H,
                    int64_t Tq, int64_t Tk, lnr_dtype dtype, void *stream);

/*
 * layernorm_fw -- LayerNorm over the last axis with mean and variance from one fused pass.
 * [L10 "Technique 2": sigma(x) = sqrt(mu(x^2) - mu(x)^2), so mu(x) and mu(x^2) come from one
 *  reduction; HW4 "Problem structure and scoring": eps inside the root, eps = 1e-8.]
 *
 *   For every row i of x [N, C]:
 *     mu = (1/C) sum_j x_ij ;  v = max((1/C) sum_j x_ij^2 - mu^2, 0)
 *     rstd = 1 / sqrt(v + eps) ;  y_ij = gamma_j * (x_ij - mu) * rstd + beta_j
 *
 *   y     [N, C] dtype, written. May equal x (in place); no other overlap.
 *   mean  [N] float32, written (mu per row), or NULL.
 *   rstd  [N] float32, written (1/sigma per row), or NULL. The backward needs both.
 *   x     [N, C] dtype, read.   gamma, beta  [C] dtype, read.
 *   eps   added to the variance inside the square root (the pages use 1e-8); must be >= 0.
 *   Limits: 1 <= C <= LNR_LAYERNORM_MAX_C; N >= 0.
 */
LNR_API int layernorm_fw(void *y, float *mean, float *rstd, const void *x, const void *gamma,
                 const void *beta, int64_t N, int64_t C, float eps, lnr_dtype dtype,
                 void *stream);

/*
 * layernorm_bw_workspace_bytes -- device workspace that layernorm_bw needs for (N, C, dtype):
 * per-block column partial sums of dgamma and dbeta. Returns 0 for an invalid shape/dtype.
 */
LNR_API size_t layernorm_bw_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype);

/*
 * layernorm_bw -- LayerNorm backward: input gradient and gamma/beta gradients.
 * [L10 "Technique 2": the input gradient rearranged into two sums computed in parallel;
 *  HW4 "Problem structure and scoring": dgamma and dbeta summed across rows.]
 *
 *   With xhat_ij = (x_ij - mean_i) * rstd_i and g_ij = gamma_j * dy_ij:
 *     dx_ij    = rstd_i * ( g_ij - (1/C) sum_k g_ik - xhat_ij * (1/C) sum_k g_ik xhat_ik )
 *     dgamma_j = sum_i dy_ij * xhat_ij ,   dbeta_j = sum_i dy_ij
 *   The row pass computes dx and accumulates per-block column partials of dgamma/dbeta in
 *   the same read of x and dy; a second kernel sums the partials in a fixed order. Column
 *   partials accumulate in float32 for fp16 storage and in float64 for fp32 storage.
 *
 *   dx      [N, C] dtype, written. Must not overlap x, dy, gamma, mean or rstd (LNR_ERR_ALIAS).
 *   dgamma, dbeta [C] dtype, written.
 *   dy, x   [N, C] dtype, read.  gamma [C] dtype, read.
 *   mean, rstd [N] float32, read: the values layernorm_fw wrote for this x.
 *   workspace  device buffer of at least layernorm_bw_workspace_bytes(N, C, dtype) bytes,
 *              16-byte aligned (LNR_ERR_ALIGN otherwise: the partial sums are written as
 *              16-byte vectors), owned by the caller; its contents on entry do not matter.
 *   Limits: 1 <= C <= LNR_LAYERNORM_MAX_C; N >= 0.
 */
LNR_API int layernorm_bw(void *dx, void *dgamma, void *dbeta, const void *dy, const void *x,
                 const void *gamma, const float *mean, const float *rstd, int64_t N,
                 int64_t C, lnr_dtype dtype, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * layernorm_bw_noalloc -- layernorm_bw for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 *   Same arguments, results, aliasing rules and errors as layernorm_bw, without the workspace:
 *   the column partials go to a device array that the library owns,
 *   LNR_NOALLOC_SCRATCH_BYTES bytes per GPU, held by every GPU the library runs on until the
 *   process ends. The call allocates nothing. Shapes whose layernorm_bw_workspace_bytes()
 *   exceeds LNR_NOALLOC_SCRATCH_BYTES return LNR_ERR_SCRATCH and enqueue nothing (at 256 or
 *   more rows: C <= 8192 for fp16, C <= 4096 for fp32).
 *   Every call on one GPU uses that GPU's one array: calls that overlap in time on one GPU
 *   (from two streams or two threads) race on it and give wrong results; calls on one stream
 *   are ordered and safe. The array keeps the last call's partials; nothing in it needs to be
 *   cleared between calls. The first call on a device looks the array's address up on that
 *   device (the device of `stream`); that call may not be under graph capture.
 */
#define LNR_NOALLOC_SCRATCH_BYTES (16u << 20)
LNR_API int layernorm_bw_noalloc(void *dx, void *dgamma, void *dbeta, const void *dy,
                                 const void *x, const void *gamma, const float *mean,
                                 const float *rstd, int64_t N, int64_t C, lnr_dtype dtype,
                                 void *stream);

/*
 * rmsnorm_fw -- RMSNorm forward: per row, one reduction of the sum of squares, then
 * y = gamma * x * rstd with rstd = 1 / sqrt(mean_j(x_j^2) + eps). No mean, no bias.
 * ["FastTransformer: Breaking the Compiler Ceiling via Architectural Co-Design", section 5.4
 *  "Vectorized Pre-RMSNorm": LayerNorm with the mean-centering removed; the page's module
 *  uses eps = 1e-6 and a learned weight only.]
 *
 *   y     [N, C] dtype, written. May equal x (in place); no other overlap.
 *   rstd  [N] float32, written (the saved statistic for rmsnorm_bw), or NULL.
 *   x     [N, C] dtype, read.   gamma  [C] dtype, read.
 *   eps   added to mean(x^2) inside the square root; must be >= 0.
 *   Limits: 1 <= C <= LNR_LAYERNORM_MAX_C; N >= 0. Same kernels, buckets and fallbacks as
 *   layernorm_fw.
 */
LNR_API int rmsnorm_fw(void *y, float *rstd, const void *x, const void *gamma, int64_t N,
                       int64_t C, float eps, lnr_dtype dtype, void *stream);

/*
 * rmsnorm_bw_workspace_bytes -- device workspace that rmsnorm_bw needs for (N, C, dtype):
 * per-block column partial sums of dgamma. Returns 0 for N = 0 and for an invalid
 * shape/dtype.
 */
LNR_API size_t rmsnorm_bw_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype);

/*
 * rmsnorm_bw -- RMSNorm backward: input gradient and gamma gradient.
 * [Same page and section as rmsnorm_fw; the gradient is the chain rule through
 *  y = gamma * x * rstd(x).]
 *
 *   With xhat_ij = x_ij * rstd_i and g_ij = gamma_j * dy_ij:
 *     dx_ij    = rstd_i * ( g_ij - xhat_ij * (1/C) sum_k g_ik xhat_ik )
 *     dgamma_j = sum_i dy_ij * xhat_ij
 *   One row reduction (the LayerNorm backward's second sum; the first, sum_k g_ik, is absent
 *   because RMSNorm subtracts no mean). Column partials and their fixed-order sum as in
 *   layernorm_bw: bitwise reproducible.
 *
 *   dx      [N, C] dtype, written. Must not overlap x, dy, gamma or rstd (LNR_ERR_ALIAS).
 *   dgamma  [C] dtype, written.
 *   dy, x   [N, C] dtype, read.  gamma [C] dtype, read.
 *   rstd    [N] float32, read: the values rmsnorm_fw wrote for this x.
 *   workspace  device buffer of at least rmsnorm_bw_workspace_bytes(N, C, dtype) bytes,
 *              16-byte aligned, owned by the caller; its contents on entry do not matter.
 *   Limits: 1 <= C <= LNR_LAYERNORM_MAX_C; N >= 0.
 */
LNR_API int rmsnorm_bw(void *dx, void *dgamma, const void *dy, const void *x, const void *gamma,
                       const float *rstd, int64_t N, int64_t C, lnr_dtype dtype, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * bdr_layernorm_fw -- bias + dropout + residual, then LayerNorm, in one pass over the rows.
 * ["CMU 11-868 L10 ...", section "Technique 1": "bias + dropout + residual" is one of the
 *  elementwise kernels between the GEMMs, and LayerNorm the reduce kernel that follows.
 *  The page gives no RNG or dropout rule: the dropout draws are an input bit mask.]
 *
 *   s_ij = residual_ij + keep_ij * (x_ij + bias_j) / (1 - p)
 *   y    = LayerNorm(s) with gamma, beta, eps (as layernorm_fw; s normalised in fp32)
 *   keep_ij = bit (j % 8) of keep_mask[i * ceil(C/8) + j / 8], least significant bit first.
 *
 *   s      [N, C] dtype, written (the residual stream); may equal residual (in place).
 *   y      [N, C] dtype, written. mean, rstd [N] float32 of s, written, or both NULL.
 *   x, residual [N, C] dtype, read. bias, gamma, beta [C] dtype, read.
 *   keep_mask [N, ceil(C/8)] bytes, read.  p  drop probability, 0 <= p < 1.
 *   Limits: 1 <= C <= LNR_LAYERNORM_MAX_C; N >= 0. C a multiple of 8 (fp16) or 4 (fp32)
 *   with every [N, C] and [C] buffer 16-byte aligned takes the vector kernel, anything else
 *   the element-wise kernel.
 */
LNR_API int bdr_layernorm_fw(void *s, void *y, float *mean, float *rstd, const void *x,
                             const void *residual, const void *bias, const uint8_t *keep_mask,
                             float p, const void *gamma, const void *beta, int64_t N, int64_t C,
                             float eps, lnr_dtype dtype, void *stream);

/*
 * bdr_layernorm_bw_workspace_bytes -- device workspace bdr_layernorm_bw needs: per-block
 * column partials of dgamma, dbeta and dbias. 0 for N = 0 or an invalid shape/dtype.
 */
LNR_API size_t bdr_layernorm_bw_workspace_bytes(int64_t N, int64_t C, lnr_dtype dtype);

/*
 * bdr_layernorm_bw -- backward of bdr_layernorm_fw from the saved s, mean and rstd.
 * [Same passage as bdr_layernorm_fw; the gradients are the chain rule through the
 *  composition, with the LayerNorm part as layernorm_bw (L10 "Technique 2").]
 *
 *   ds        = LayerNorm input gradient of dy (as layernorm_bw) + ds_extra
 *   dresidual = ds,   dx = keep * ds / (1 - p),   dbias_j = sum_i dx_ij,
 *   dgamma_j = sum_i dy_ij * shat_ij,   dbeta_j = sum_i dy_ij,  shat = (s - mean) * rstd.
 *
 *   dresidual, dx [N, C] dtype, written; dresidual may equal dy or ds_extra (in place); dx
 *   overlaps nothing.  dgamma, dbeta, dbias [C] dtype, written.
 *   dy, s [N, C] dtype, read.  ds_extra [N, C] dtype, read, or NULL (no other path into s).
 *   keep_mask, p as in the forward.  gamma [C] dtype; mean, rstd [N] float32, read.
 *   workspace  bdr_layernorm_bw_workspace_bytes(N, C, dtype) bytes, 16-byte aligned, caller
 *   owned; contents on entry do not matter; must not overlap any other argument.
 *   Limits and the choice of kernel as in the forward.
 */
LNR_API int bdr_layernorm_bw(void *dresidual, void *dx, void *dgamma, void *dbeta, void *dbias,
                             const void *dy, const void *ds_extra, const void *s,
                             const uint8_t *keep_mask, float p, const void *gamma,
                             const float *mean, const float *rstd, int64_t N, int64_t C,
                             lnr_dtype dtype, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * attn_softmax_fw_skip / attn_softmax_bw_skip -- attn_softmax_fw / attn_softmax_bw that do not
 * read score vectors whose keys are all masked.
 * [HW4 "Problem structure and scoring": future tokens and padded keys are -inf, so their
 *  probabilities are exactly 0; FastTransformer section 3 "The Surprising Bottleneck": the
 *  materialised probability tensor's HBM traffic is the attention cost.]
 *
 *   Same arguments, layout, limits, aliasing and errors as attn_softmax_fw, and for the
 *   backward as attn_softmax_bw plus the forward's mask and causal flag. A 16-byte run of a
 *   row (8 fp16 or 4 fp32 elements) whose keys all lie after the query (causal) or all carry a
 *   -inf mask entry is not read: the forward takes its scores as -inf and writes its zeros;
 *   the backward writes zeros there without reading y or dy. Every element of the outputs is
 *   written.
 *   Results equal attn_softmax_fw's (forward) when the skipped scores are finite, and
 *   attn_softmax_bw's (backward, up to the sign of zero) when out_fw is 0 and dout is finite at
 *   the skipped positions -- which holds when out_fw is the forward's output for the same mask
 *   and causal flag. Rows whose byte length is not a multiple of 16, or buffers not 16-byte
 *   aligned, run the dense entry points (no skipping, same results).
 *   Only exact -inf mask entries are skipped; a large finite negative mask is read as usual.
 */
LNR_API int attn_softmax_fw_skip(void *out, const void *inp, const void *mask, int64_t B,
                                 int64_t H, int64_t Tq, int64_t Tk, int causal, lnr_dtype dtype,
                                 void *stream);
LNR_API int attn_softmax_bw_skip(void *dinp, const void *dout, const void *out_fw,
                                 const void *mask, int64_t B, int64_t H, int64_t Tq, int64_t Tk,
                                 int causal, lnr_dtype dtype, void *stream);

/*
 * cross_entropy_fw_workspace_bytes -- device workspace cross_entropy_fw needs for (N, V,
 * dtype): per-chunk partial (max, sum) pairs when rows are longer than 256 KB (V above 65536
 * fp32 or 131072 fp16 logits) and there are too few of them to fill the GPU, so that each row
 * is split over several workgroups; 0 when rows are not split (every shorter row, and the
 * common case of thousands of rows) and for an invalid shape/dtype.
 */
LNR_API size_t cross_entropy_fw_workspace_bytes(int64_t N, int64_t V, lnr_dtype dtype);

/*
 * cross_entropy_fw -- softmax cross-entropy over a vocabulary, per row.
 * ["CMU 11-868 L10 ...", section "Technique 1": cross entropy is one of the custom reduce
 *  kernels; the inference section: a softmax over the whole vocabulary. No formula is
 *  printed; this is the textbook one, without label smoothing.]
 *
 *   lse_i  = log sum_j exp(z_ij)          (one streaming pass over the row)
 *   loss_i = lse_i - z_i,target_i
 *   loss   [N] float32, written.  lse [N] float32, written (saved for cross_entropy_bw).
 *   logits [N, V] dtype, read; any V >= 1 (odd V included; rows need not be 16-byte aligned).
 *   target [N] int64, read: a class in [0, V), or ignore_index (loss 0). Any other value
 *          gives loss NaN for that row (the kernel cannot raise an error).
 *   workspace  cross_entropy_fw_workspace_bytes(N, V, dtype) bytes (may be NULL when that
 *          is 0), 8-byte aligned, owned by the caller; contents on entry do not matter.
 *   Limits: N <= INT32_MAX, 1 <= V <= INT32_MAX / 2.
 */
LNR_API int cross_entropy_fw(float *loss, float *lse, const void *logits, const int64_t *target,
                             int64_t N, int64_t V, int64_t ignore_index, lnr_dtype dtype,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * cross_entropy_bw -- gradient of sum_i scale * dloss_i * loss_i with respect to the logits.
 * [Same passages as cross_entropy_fw; the derivative of lse - z_t is softmax - onehot.]
 *
 *   dlogits_ij = scale * dloss_i * ( exp(z_ij - lse_i) - [j == target_i] )
 *   dlogits [N, V] dtype, written; may equal logits (in place), no other overlap.
 *   logits  [N, V] dtype, read.  target [N] int64, read.
 *   lse     [N] float32, read: the values cross_entropy_fw wrote.
 *   dloss   [N] float32 upstream gradient of each row's loss, or NULL for all ones.
 *   scale   a finite factor on every row (for a mean over rows: 1 / number of rows counted).
 *   Rows whose target is ignore_index get a zero gradient row; any other target outside
 *   [0, V) gives a row of NaN.
 */
LNR_API int cross_entropy_bw(void *dlogits, const void *logits, const int64_t *target,
                             const float *lse, const float *dloss, float scale, int64_t N,
                             int64_t V, int64_t ignore_index, lnr_dtype dtype, void *stream);

/*
 * lnr_copy -- measurement helper, not part of the method: copies `bytes` bytes from src to
 * dst with the same 128-bit load/store pattern as the row kernels, giving the achievable
 * streaming ceiling that the kernels' bandwidth is compared with. dst and src must not
 * overlap; bytes must be a multiple of 16 and both pointers 16-byte aligned.
 */
LNR_API int lnr_copy(void *dst, const void *src, size_t bytes, void *stream);

/*
 * lnr_xor2 -- measurement helper, not part of the method: writes dst = a XOR b over `bytes`
 * bytes, reading two buffers and writing one (the traffic pattern of both backward kernels)
 * with the same 128-bit non-temporal accesses as lnr_copy. It gives the achievable streaming
 * ceiling for that pattern at a given size. dst must not overlap a or b (a and b may be the
 * same buffer); bytes must be a multiple of 16 and all pointers 16-byte aligned.
 */
LNR_API int lnr_xor2(void *dst, const void *a, const void *b, size_t bytes, void *stream);

/*
 * lnr_time_next_launch -- measurement helper, not part of the method: the next kernel that
 * the calling thread launches through this library records `start_event` when that kernel
 * begins and `stop_event` when it ends (both hipEvent_t, created by the caller with timing
 * enabled), so hipEventElapsedTime gives that kernel's own duration without the dispatch
 * latency an event recorded before the call would include. Only the next launch is timed,
 * then the request is cleared; for an operation of two kernels (layernorm_bw) that is the
 * first kernel. Both NULL cancels a pending request; exactly one NULL is LNR_ERR_NULL.
 * Per-thread state; touches no device until the timed launch.
 */
LNR_API int lnr_time_next_launch(void *start_event, void *stop_event);

/*
 * lnr_softmax_plan -- introspection of the row-length dispatch (the compile-time template
 * choice at launch that the L10 lecture's "Technique 2" describes and the HW4 page's
 * softmax backward asks for): for rows of Tk elements of `dtype` in 16-byte-aligned
 * buffers, writes the bucket (the longest row of the chosen instantiation; 0 = element-wise
 * fallback), the lanes per row and the 16-byte vectors per lane of the forward (which = 0)
 * or backward (which = 1) kernel, or of the read-skipping forward (2) or backward (3), which
 * call the dense kernels for rows that are not whole 16-byte vectors. `which` outside 0..3
 * is LNR_ERR_SHAPE. Touches no device.
 */
LNR_API int lnr_softmax_plan(int64_t Tk, lnr_dtype dtype, int which, int *bucket,
                             int *lanes_per_row, int *vectors_per_lane);

/*
 * lnr_layernorm_plan -- the same for LayerNorm rows of C elements: `which` = 0 for the
 * forward kernel, 1 for the backward row kernel. Also writes the workgroup size and the
 * number of workgroups (for the backward: the number of dgamma/dbeta partial rows) that a
 * call with N rows launches. Touches no device.
 */
LNR_API int lnr_layernorm_plan(int64_t N, int64_t C, lnr_dtype dtype, int which, int *bucket,
                       int *lanes_per_row, int *vectors_per_lane, int *workgroup,
                       int64_t *blocks);

/* lnr_strerror -- static text for an lnr_status value (never NULL). */
LNR_API const char *lnr_strerror(int status);

/* lnr_build_info -- static text naming the target architecture and library version. */
LNR_API const char *lnr_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* LNR_H */
