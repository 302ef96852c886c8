/*
 * path_attn.h -- C ABI of the PaTH attention library for AMD MI355X (gfx950).
 *
 * PaTH attention (sources, by page title and section):
 *   [TS]  "技術要約: PaTH Attention" (gist.science, Japanese technical summary of
 *         arXiv 2505.16381), section 2 "手法": attention logit
 *         k_j^T (prod_{s=j+1..i} H_s) q_i with H_s = I - beta_s w_s w_s^T and
 *         beta_s = 2 sigmoid(.) in (0, 2); section 3 "効率的な学習と推論": UT-
 *         transform form of a product of H's, a blockwise FlashAttention-style
 *         algorithm (boundary-adjusted queries/keys, right-to-left scan over
 *         key blocks), and decoding by updating cached keys in place with the
 *         newest H_t; section 6 "限界": beta is clipped near 2 for bf16.
 *   [IPX] "거리에서 경로로, PaTH Attention" (iplexlaw.co.kr), section 3
 *         (softmax over the transformed scores, weighted sum of values) and
 *         section 4 (PaTH-FoX: an additive, data-dependent forget gate).
 *
 * All functions are synchronous on the host: argument errors are reported
 * before anything is enqueued.  Kernels run asynchronously on `stream`
 * (path_stream_t is hipStream_t, declared here without the HIP headers;
 * NULL = the default stream) and results are valid once that stream's work
 * has completed.  The library keeps no pointer after a
 * call returns, allocates no device memory and holds no mutable global
 * state; calls from several host threads are safe (calls that share output
 * or workspace memory must be ordered by the caller).
 *
 * Layout: every tensor is contiguous and row-major.  Per-token tensors are
 * [B, H, L, d] (B batches, H heads, L tokens, head dimension d); per-token
 * scalars are [B, H, L].  Pointers are DEVICE pointers owned by the caller
 * and must be 16-byte aligned.  d must be 64 or 128 (other head sizes
 * return PATH_EUNSUPPORTED).  Any L >= 1 is accepted.
 *
 * Numerics: dtype selects the element type of q, k, v, w, the output and the
 * caches.  beta, the log-forget gate, lse and all accumulation are fp32.
 * PATH_DTYPE_F32 runs fp32 end to end (fp32 matrix-core instructions);
 * PATH_DTYPE_BF16 feeds bf16 operands to the matrix cores and accumulates in
 * fp32.  w is used as given (not re-normalised) and beta is not clipped; NaN
 * or Inf inputs propagate and are not checked.
 */
#ifndef PATH_ATTN_H
#define PATH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ABI version.  It changes only when an existing entry point changes its
 * parameters or meaning; new capabilities come as new entry points (the
 * _ex variants), which leave it unchanged.
 */
#define PATH_ABI_VERSION 1

/* The HIP stream type: hipStream_t is `struct ihipStream_t *`, so a
 * hipStream_t converts to this type without a cast. */
typedef struct ihipStream_t *path_stream_t;

typedef enum {
    PATH_OK = 0,
    PATH_EINVAL = 1,        /* NULL pointer, bad size, misaligned, workspace too small, n > ncap */
    PATH_EUNSUPPORTED = 2,  /* valid but not implemented (head dimension other than 64, 128) */
    PATH_EHIP = 3,          /* the HIP runtime rejected a launch */
    PATH_ESCRATCH = 4       /* path_decode_step_noalloc: the problem needs more than its fixed scratch */
} path_status_t;

typedef enum {
    PATH_DTYPE_F32 = 0,
    PATH_DTYPE_BF16 = 1
} path_dtype_t;

/* Version of this ABI (PATH_ABI_VERSION). */
int path_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *path_status_string(path_status_t status);

/*
 * Workspace bytes that path_attn_fwd needs for these sizes (0 if the sizes
 * are invalid).  The caller allocates it on the device; its contents on
 * entry do not matter and are garbage afterwards.
 */
size_t path_attn_fwd_workspace_size(int B, int H, int L, int d, path_dtype_t dtype);

/*
 * Causal PaTH attention forward ([TS] s.2 logit, [IPX] s.3 softmax and value
 * sum, [TS] s.3 blockwise algorithm), with the optional PaTH-FoX bias
 * ([IPX] s.4):
 *
 *   s_ij = scale * k_j^T (H_{j+1} H_{j+2} ... H_i) q_i  +  sum_{s=j+1..i} logf_s,
 *          j <= i,  H_s = I - beta_s w_s w_s^T
 *   out_i = sum_{j<=i} softmax_j(s_ij) v_j,   lse_i = log sum_{j<=i} exp(s_ij)
 *
 * q, k, v, w : [B, H, L, d], element type `dtype`           (read only)
 * beta       : [B, H, L] fp32                                (read only)
 * logf       : [B, H, L] fp32 log forget gate, or NULL for plain PaTH.
 *              The bias is added after `scale`, and is 0 on the diagonal.
 * out        : [B, H, L, d], element type `dtype`            (written; must not alias an input)
 * lse        : [B, H, L] fp32 natural-log normaliser, or NULL
 * scale      : multiplies the transformed dot product; <= 0 selects 1/sqrt(d)
 * workspace  : device scratch of at least path_attn_fwd_workspace_size() bytes
 *
 * Returns PATH_OK, PATH_EINVAL, PATH_EUNSUPPORTED or PATH_EHIP.
 */
path_status_t path_attn_fwd(const void *q, const void *k, const void *v, const void *w, const float *beta,
                            const float *logf, void *out, float *lse, int B, int H, int L, int d,
                            path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                            path_stream_t stream);

/*
 * path_attn_fwd with options.  flags is a bitwise OR of:
 *
 *   PATH_FWD_SKIP_NEGLIGIBLE  with logf: stop the right-to-left walk over key
 *       blocks for a query block once every remaining block provably adds
 *       less than 2^-64 of the running softmax maximum per key, i.e. far
 *       below fp32 resolution of the output.  The bound is
 *       ||qhat_i|| * max_j ||k_j|| + (forget-gate bias of the block boundary),
 *       valid because every transition is a contraction when
 *       0 <= beta_s ||w_s||^2 <= 2 (blocks violating that are never skipped).
 *       The forget gate makes old keys decay, so long sequences need only a
 *       window of recent blocks ([IPX] s.4).  Ignored without logf.
 *
 * Other bits must be zero (PATH_EINVAL).  Arguments and errors otherwise as
 * path_attn_fwd, which is path_attn_fwd_ex with flags = 0.
 */
#define PATH_FWD_SKIP_NEGLIGIBLE 1u
path_status_t path_attn_fwd_ex(const void *q, const void *k, const void *v, const void *w, const float *beta,
                               const float *logf, void *out, float *lse, int B, int H, int L, int d,
                               path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                               unsigned flags, path_stream_t stream);

/*
 * PaTH forward with the producer of w and beta fused into it.
 *
 * Source: "거리에서 경로로, PaTH Attention" (iplexlaw.co.kr), section 3, and the
 * Chinese summary's method paragraph: w comes from a low-dimensional linear
 * projection, a short convolution of width 3 and an L2 normalisation, and
 * beta = 2 sigmoid(.) ("技術要約: PaTH Attention", section 2: beta_s =
 * 2 sigmoid(u^T x_s + b)).  The projections are plain matrix products done by
 * the caller; this call takes their outputs and does the rest inside the
 * prep kernel, so w and beta never go through device memory:
 *   y_t[c]  = sum_{tau=0..2} conv_w[h][c][tau] * wraw[b][h][t-2+tau][c]
 *             (causal, per channel, zero before the first token)
 *   w_t     = y_t / max(||y_t||, 1e-12)
 *   beta_t  = 2 sigmoid(zbeta[b][h][t]), capped at beta_clip when beta_clip > 0
 * and then exactly path_attn_fwd on (q, k, v, w, beta, logf).  (The kernel
 * keeps y_t, rounded to the element type, and uses beta_t / max(||y_t||^2,
 * 1e-24) instead, which gives the same transition matrices.)
 *
 *   wraw    [B, H, L, d] element type, 16-byte aligned (the role of w above)
 *   conv_w  [H, d, 3] fp32, 16-byte aligned
 *   zbeta   [B, H, L] fp32 (the role of beta above)
 *   beta_clip  0 for no cap, else a cap in (0, 2]; negative or non-finite
 *              values are rejected
 * Every other argument, the workspace and the errors are those of
 * path_attn_fwd (wraw and zbeta are checked like w and beta; conv_w must not
 * overlap out, lse or the workspace).  Device pointers, owned by the caller.
 */
path_status_t path_attn_fwd_fused(const void *q, const void *k, const void *v, const void *wraw,
                                  const float *conv_w, const float *zbeta, float beta_clip, const float *logf,
                                  void *out, float *lse, int B, int H, int L, int d, path_dtype_t dtype, float scale,
                                  void *workspace, size_t workspace_bytes, path_stream_t stream);

/*
 * The two stages of path_attn_fwd, for callers that schedule or time them
 * separately (path_attn_fwd is exactly prep followed by scan on one stream).
 *
 * path_attn_fwd_prep: per 64-token block, the UT transform of the block's
 *   transitions ([TS] s.3), the boundary-adjusted queries and keys, the
 *   block's transition product and the causal attention inside the block.
 *   Same arguments and errors as path_attn_fwd.  After it, rows of the first
 *   block are final; other rows of out/lse hold intermediate values.
 * path_attn_fwd_scan: the right-to-left scan over earlier key blocks with
 *   online softmax ([TS] s.3), finishing out and lse.  `workspace` must hold
 *   the results of a path_attn_fwd_prep call with the same sizes, dtype,
 *   scale, out and lse, enqueued before it on the same stream (or otherwise
 *   completed); has_logf must be non-zero iff that call had a logf.
 */
path_status_t path_attn_fwd_prep(const void *q, const void *k, const void *v, const void *w, const float *beta,
                                 const float *logf, void *out, float *lse, int B, int H, int L, int d,
                                 path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                                 path_stream_t stream);
path_status_t path_attn_fwd_scan(void *out, float *lse, int has_logf, int B, int H, int L, int d,
                                 path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                                 path_stream_t stream);

/* Workspace bytes that path_decode_step needs (0 if the sizes are invalid). */
size_t path_decode_workspace_size(int B, int H, int64_t n, int d, path_dtype_t dtype);

/*
 * One PaTH decode step ([TS] s.3, inference): the newest transition
 * H_t = I - beta_t w_t w_t^T is applied IN PLACE to every cached key,
 *
 *   kcache[b,h,j,:] <- H_t kcache[b,h,j,:]      for j in [0, n)
 *
 * (rounded to `dtype`), so that no w/beta history is kept; then the single
 * query q_t attends to the cache with softmax.  If k_new and v_new are both
 * non-NULL they are stored at row n AFTER the update (the newest key has the
 * empty product) and the query attends to n+1 rows; otherwise to n rows.
 *
 * kcache, vcache : [B, H, ncap, d] element type `dtype`; rows >= n (+1) untouched
 * n              : rows in use, 0 <= n <= ncap (n + 1 <= ncap with k_new; at least one row must attend)
 * q, w           : [B, H, d] element type `dtype`; beta: [B, H] fp32
 * k_new, v_new   : [B, H, d] or both NULL
 * out            : [B, H, d] element type `dtype`; lse: [B, H] fp32 or NULL
 * scale          : <= 0 selects 1/sqrt(d)
 * workspace      : at least path_decode_workspace_size(B, H, n (+1), d, dtype) bytes
 *
 * A cache row that went through steps j+1..t holds H_t ... H_{j+1} k_j; as
 * every H is symmetric its dot product with q_t equals the forward logit
 * k_j^T (H_{j+1} ... H_t) q_t.  Buffers must not overlap (PATH_EINVAL).
 */
path_status_t path_decode_step(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q, const void *w,
                               const float *beta, const void *k_new, const void *v_new, void *out, float *lse,
                               int B, int H, int d, path_dtype_t dtype, float scale, void *workspace,
                               size_t workspace_bytes, path_stream_t stream);

/*
 * path_decode_step with the PaTH-FoX forget gate ([IPX] s.4): with logf and
 * fcache (both or neither; both NULL is exactly path_decode_step) row j's
 * logit gets sum_{s=j+1..t} log f_s = c_t - c_j, where fcache holds
 * c_j = sum_{s<=j} log f_s for the cached rows and c_t = c_{n-1} + logf_t
 * (c_{-1} = 0); with k_new, c_t is stored at fcache row n.
 *
 * logf           : [B, H] fp32 log f_t of the current token, or NULL
 * fcache         : [B, H, ncap] fp32 gate cache (rows [0, n) read, row n written with k_new), or NULL
 * Every other argument, the workspace and the errors are those of
 * path_decode_step.
 */
path_status_t path_decode_step_ex(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q, const void *w,
                                  const float *beta, const float *logf, float *fcache, const void *k_new,
                                  const void *v_new, void *out, float *lse, int B, int H, int d, path_dtype_t dtype,
                                  float scale, void *workspace, size_t workspace_bytes, path_stream_t stream);

/*
 * Workspace bytes that path_decode_step_fused needs (0 if the sizes are
 * invalid): those of path_decode_workspace_size plus room for the step's w and
 * beta.  n as for path_decode_workspace_size (the attending rows).
 */
size_t path_decode_fused_workspace_size(int B, int H, int64_t n, int d, path_dtype_t dtype);

/*
 * path_decode_step_ex with the producer of w and beta fused into it: the
 * decode counterpart of path_attn_fwd_fused ("거리에서 경로로, PaTH
 * Attention", section 3: w from a projection, a short convolution of width 3
 * and an L2 normalisation; "技術要約: PaTH Attention", section 2: beta =
 * 2 sigmoid(.)).  For the current token t, with x the rows of raw projection
 * outputs (the role of wraw in path_attn_fwd_fused):
 *   y_t[c]  = sum_{tau=0..2} conv_w[h][c][tau] * x_{t-2+tau}[c]
 *             (x_t = wraw; x_{t-2}, x_{t-1} from conv_state)
 *   w_t     = y_t / max(||y_t||, 1e-12)
 *   beta_t  = 2 sigmoid(zbeta), capped at beta_clip when beta_clip > 0
 * and then exactly path_decode_step_ex with (w_t, beta_t).  As in the forward,
 * the kernels use y_t rounded to the element type with beta_t / max(||y_t||^2,
 * 1e-24), which gives the same transition.  conv_state then moves on by one
 * token: it holds (x_{t-1}, x_t) for the next step.
 *
 *   wraw        [B, H, d] element type, 16-byte aligned: the current token's raw row
 *   conv_w      [H, d, 3] fp32, 16-byte aligned (as in path_attn_fwd_fused)
 *   zbeta       [B, H] fp32
 *   beta_clip   0 for no cap, else a cap in (0, 2]; negative or non-finite
 *               values are rejected
 *   conv_state  [B, H, 2, d] element type, 16-byte aligned, read and written:
 *               the raw rows of the two previous tokens, oldest first (zero rows
 *               before the first token; after a prefix of L tokens, its rows L-2
 *               and L-1)
 *   workspace   at least path_decode_fused_workspace_size(B, H, n (+1), d, dtype) bytes
 * Every other argument, the results and the errors are those of
 * path_decode_step_ex.  conv_state must not overlap any other buffer, and
 * wraw, conv_w and zbeta no buffer the step writes (PATH_EINVAL).  Device
 * pointers, owned by the caller.
 */
path_status_t path_decode_step_fused(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q,
                                     const void *wraw, const float *conv_w, const float *zbeta, float beta_clip,
                                     void *conv_state, const float *logf, float *fcache, const void *k_new,
                                     const void *v_new, void *out, float *lse, int B, int H, int d,
                                     path_dtype_t dtype, float scale, void *workspace, size_t workspace_bytes,
                                     path_stream_t stream);

/*
 * path_decode_step_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: the split partials go to a fixed scratch
 * array of path_decode_noalloc_max_bytes() bytes (32 MiB) that the library
 * holds on every device it runs on until the process ends, and the call itself
 * allocates nothing.  Every call on one device shares that device's array, so
 * calls that overlap in time on one device (other streams, other host threads)
 * race; calls ordered on one stream are safe.  Nothing in the array needs to
 * start at zero (every split writes its whole record before the merge reads
 * it).  The scratch a call needs is path_decode_workspace_size(B, H, n (+1),
 * d, dtype); larger problems return PATH_ESCRATCH (before anything is
 * enqueued: B * H above 127 100 at d = 64 or 64 527 at d = 128).  The first call on
 * a device looks the array's address up on that device (the current device).
 * Arguments, results and the other errors are those of path_decode_step_ex.
 */
size_t path_decode_noalloc_max_bytes(void);
path_status_t path_decode_step_noalloc(void *kcache, void *vcache, int64_t n, int64_t ncap, const void *q,
                                       const void *w, const float *beta, const float *logf, float *fcache,
                                       const void *k_new, const void *v_new, void *out, float *lse, int B, int H,
                                       int d, path_dtype_t dtype, float scale, path_stream_t stream);

/*
 * Decode cache of a prefix from its forward pass ([TS] s.3: prefill, then
 * decode with in-place key updates).  After path_attn_fwd (or
 * path_attn_fwd_prep) has processed tokens 0 .. L-1, this fills the caches
 * that L decode steps would have produced:
 *
 *   kcache[b,h,j,:] = H_{L-1} ... H_{j+1} k_j     (H_{j+1} applied first; row L-1 = k_{L-1})
 *   vcache[b,h,j,:] = v_j                          for j in [0, L)
 *   fcache[b,h,j]   = sum_{s<=j} logf[b,h,s]        (when logf and fcache are given)
 *
 * rounded to `dtype`, so that path_decode_step with n = L continues the
 * sequence.  The keys come from the boundary-adjusted key blocks and block
 * transition products that the forward pass left in its workspace.
 *
 * workspace      : the workspace of a path_attn_fwd / path_attn_fwd_prep call with
 *                  the same B, H, L, d and dtype, enqueued before this call on the
 *                  same stream (or completed); results are undefined otherwise
 * v              : [B, H, L, d] element type `dtype`, the prefix values (read only)
 * logf, fcache   : [B, H, L] fp32 prefix log-forget gate and [B, H, ncap] fp32 gate cache
 *                  for a PaTH-FoX decode, or both NULL
 * kcache, vcache : [B, H, ncap, d] element type `dtype`, ncap >= L; rows >= L untouched
 *
 * Returns PATH_OK, PATH_EINVAL (NULL, sizes, misaligned, workspace too small,
 * ncap < L, overlapping buffers), PATH_EUNSUPPORTED or PATH_EHIP.
 */
path_status_t path_decode_cache_from_fwd(const void *workspace, size_t workspace_bytes, const void *v,
                                         const float *logf, void *kcache, void *vcache, float *fcache,
                                         int64_t ncap, int B, int H, int L, int d, path_dtype_t dtype,
                                         path_stream_t stream);

/*
 * Workspace bytes for path_attn_bwd (0 if the sizes are invalid or not
 * supported): enough to process all B*H heads at once when that takes at most
 * 32 GiB, else the largest whole number of heads that fits in 32 GiB (at least
 * one).  path_attn_bwd_workspace_size(1, 1, L, d, dtype) is one head's share;
 * path_attn_bwd accepts any workspace of at least one share and processes
 * floor(workspace_bytes / share) heads at a time (results do not depend on it).
 * One share is 3 * 64 * d element-type values (2 * 64 * d for bf16) per pair
 * of 64-token blocks (nb (nb - 1) / 2 pairs, nb = ceil(L / 64)) plus 4.3 KiB
 * (d = 64, bf16) to 10.5 KiB (d = 128, fp32) per token: 48.6 MiB per head at
 * L = 4096, d = 64, bf16; 95.2 MiB at d = 128, bf16.
 */
size_t path_attn_bwd_workspace_size(int B, int H, int L, int d, path_dtype_t dtype);

/*
 * Backward pass of path_attn_fwd: gradients of
 *     loss = sum_{b,h,i} dout_i . out_i  +  sum_{b,h,i} dlse_i lse_i
 * with respect to q, k, v, w, beta and (with the forget gate) logf.  The pages
 * give the blockwise algorithm ([TS] s.3) as what makes PaTH trainable and
 * print no gradient; this is the chain rule applied to the forward's definition
 * (path_attn_fwd above), evaluated on the same 64-token blocks: a walk over
 * key blocks per query block for the query side, one per key block for the
 * key side and the block transitions, and a per-block pass through the UT
 * transform.  The walks run on the matrix cores in `dtype` (bf16 operands
 * with fp32 accumulation for bf16, fp32 for fp32); the per-block passes on
 * the matrix cores too, with fp32 operands for fp32 and, for bf16, bf16
 * operands where they are input values and hi + lo bf16 pairs (about 16
 * significant bits) for the derived fp32 matrices.
 *
 * q, k, v, w, out, dout : [B, H, L, d] element type `dtype` (read only); out is the
 *                         forward's output for these inputs
 * beta, lse             : [B, H, L] fp32 (read only); lse is the forward's natural-log
 *                         normaliser (path_attn_fwd's lse output)
 * logf, dlogf           : [B, H, L] fp32 log forget gate and its gradient, or both NULL
 * dlse                  : [B, H, L] fp32 gradient with respect to lse, or NULL (zero)
 * dq, dk, dv, dw        : [B, H, L, d] element type `dtype` (written)
 * dbeta                 : [B, H, L] fp32 (written)
 * scale                 : as in path_attn_fwd (<= 0 selects 1/sqrt(d))
 * workspace             : device scratch, see path_attn_bwd_workspace_size
 *
 * d must be 64 or 128.  Outputs must not overlap each
 * other, the inputs or the workspace.  Returns PATH_OK, PATH_EINVAL (NULL,
 * sizes, misaligned, workspace below one head's share, overlaps),
 * PATH_EUNSUPPORTED or PATH_EHIP.
 */
path_status_t path_attn_bwd(const void *q, const void *k, const void *v, const void *w, const float *beta,
                            const float *logf, const void *out, const float *lse, const void *dout,
                            const float *dlse, void *dq, void *dk, void *dv, void *dw, float *dbeta, float *dlogf,
                            int B, int H, int L, int d, path_dtype_t dtype, float scale, void *workspace,
                            size_t workspace_bytes, path_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PATH_ATTN_H */
