/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library.
 *
 * Two operations, both asynchronous on the caller's HIP stream (each also with
 * grouped-query heads, the _gqa calls; the forward also with strides and a
 * 16-bit O, fa_fwd_ex), the forward's backward (fa_bwd), and the paged cache's
 * append kernel and host page allocator (fa_kv_append, fa_pager_*), and the
 * pre-LayerNorm attention block around the forward (fa_ln_*, fa_linear,
 * fa_prenorm_attention):
 *
 *   fa_fwd           exact attention forward: O = softmax(scale * Q K^T + mask) V
 *                    and the per-row log-sum-exp, computed tile by tile with an
 *                    online softmax so that the Nq x Nk score matrix never
 *                    exists in memory.  Definition: Kernel-Inference-Engine
 *                    page, attention-block chart (softmax(QK^T/sqrt(d))) and
 *                    tile dataflow chart (S = Q_i K_j^T scale, mask, online
 *                    softmax with running max and normaliser, rescale of the
 *                    O accumulator, O += P V_j, normalise and store); masks
 *                    as on the gpu-inference page, section 02 (causal mask
 *                    combined with the padding mask before the softmax);
 *                    the saved log-sum-exp statistic of that same section.
 *
 *   fa_decode_paged  one query per (sequence, head) attending to every cached
 *                    token of its sequence, the cache stored in fixed-size
 *                    pages found through a page table (inference kernel
 *                    cookbook page, recipe 03 "Paged Attention"; NanoInfer
 *                    page, paged KV-cache allocator).  Same definition with
 *                    query length 1.
 *
 * Conventions (after the Kernel-Inference-Engine page's op sequence chart:
 * the framework allocates outputs and workspace, raw device pointers plus the
 * stream go to the launch, no host round trip, no private allocation, error
 * read back right after the launch; and its design note that the op has no
 * CPU kernel):
 *   - Every pointer is a DEVICE pointer owned by the caller (except the
 *     host-side page allocator, fa_pager_*).  The kernels' entry points never
 *     allocate, free, copy to/from the host or synchronise.
 *   - `stream` is a hipStream_t passed as void*; NULL = the null stream.
 *   - Calls return once the kernels are enqueued.  Faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - Argument checks all happen before any HIP call, so a rejected call
 *     has no side effect.  Values that live in device memory (kv_lens,
 *     page_table) cannot be checked without a sync: kernels clamp them into
 *     range so that they never read or write outside the buffers whose sizes
 *     the arguments describe; results for out-of-contract values are
 *     unspecified.
 *   - Results are a pure function of the inputs: bitwise reproducible from
 *     run to run.
 *   - Thread safety: calls may be made concurrently from several threads.
 *     fa_last_hip_error() is per thread.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FA_OK 0
#define FA_ERR_NULL 1        /* a required pointer is NULL */
#define FA_ERR_SHAPE 2       /* a size is negative, or a product overflows the index range */
#define FA_ERR_UNSUPPORTED 3 /* head dim, page size or dtype not built */
#define FA_ERR_ALIGN 4       /* a pointer is not aligned as stated below */
#define FA_ERR_WORKSPACE 5   /* workspace missing or smaller than fa_decode_workspace_bytes */
#define FA_ERR_HIP 6         /* a HIP launch failed; see fa_last_hip_error() */
#define FA_ERR_ARG 7         /* scale not finite and > 0, causal not 0/1, or eps not finite and >= 0 */
#define FA_ERR_NOMEM 8       /* the page allocator has too few free pages */
#define FA_ERR_SCRATCH 9     /* fa_decode_paged_noalloc: the problem needs more than its fixed scratch */

/* element types of Q, K, V (and the KV pools); FA_DTYPE_F32 only for fa_fwd_ex's O */
#define FA_DTYPE_F16 0
#define FA_DTYPE_BF16 1
#define FA_DTYPE_F32 2

/*
 * Exact attention forward.
 *
 *   q        [B, H, Nq, d]  f16/bf16 (dtype), contiguous, d innermost; 16-byte aligned
 *   k, v     [B, H, Nk, d]  same dtype and layout; 16-byte aligned
 *   o        [B, H, Nq, d]  float32 output (written); 16-byte aligned
 *   lse      [B, H, Nq]     float32 output (written): natural log of the sum of
 *                           exp(scaled scores) over the row's valid keys;
 *                           4-byte aligned
 *   d        a multiple of 8 from 8 to 128 (the Kernel-Inference-Engine page's
 *            head-dim templates 32, 64, 80, 96, 128 among them)
 *   scale    multiplies Q.K (finite, > 0; typically 1/sqrt(d))
 *   causal   0 or 1.  Query row i may see key j only if j <= i + (Nk - Nq)
 *            (aligned at the bottom-right; plain lower-triangular when Nq == Nk)
 *   kv_lens  NULL (all Nk keys valid) or a device int32 [B]: keys j >= kv_lens[b]
 *            are masked for every head and query row of batch b.  Values are
 *            clamped to [0, Nk].
 *
 * A row with no valid key gets O = 0 and LSE = -inf.  B, H or Nq of 0 is an
 * empty problem (FA_OK, nothing written, pointers may be NULL).  Nk = 0 is
 * allowed (every row empty).  The keys of one (b, h) are addressed with
 * 32-bit byte offsets: (Nk + 64) * d * 2 must stay below 2^31, else
 * FA_ERR_SHAPE.  The library needs no workspace for this call.
 *
 * Two kernels compute this: a tiled one (a workgroup per 128-row query tile)
 * and, when that would launch fewer than 256 workgroups (few heads, short or
 * single sequences) and d > 96 or d <= 64, a split-key one (a workgroup per
 * 32-row block whose four waves share out its keys and merge their partial
 * results by the log-sum-exp rule; eight waves when the tiled grid would be at
 * most 64 workgroups and d <= 64).  All give the same result up to rounding
 * order.  The environment variable FA_FWD_SPLIT=0, 1 or 8, read at each call,
 * forces the tiled kernel or the split-key kernel with four or eight waves (for
 * testing each on any shape; eight becomes four above d = 64).
 */
int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H,
           int Nq, int Nk, int d, float scale, int causal, const int32_t *kv_lens, int dtype,
           void *stream);

/*
 * fa_fwd with grouped-query heads (multi-query and grouped-query attention,
 * the head-sharing variants of the llm-kernel-lib page's "Ablation Study"):
 *
 *   k, v     [B, H_kv, Nk, d]; H must be a positive multiple of H_kv.  Query
 *            head h reads K/V head h / (H / H_kv): consecutive query heads
 *            share one K/V head.  H_kv = H is fa_fwd; H_kv = 1 is multi-query.
 *
 * Every other argument, layout, alignment and error as for fa_fwd; H_kv < 1
 * or H not a multiple of H_kv (with H > 0) is FA_ERR_SHAPE.
 */
int fa_fwd_gqa(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H,
               int H_kv, int Nq, int Nk, int d, float scale, int causal, const int32_t *kv_lens,
               int dtype, void *stream);

/*
 * fa_fwd_gqa with explicit strides and a choice of O's element type, for
 * tensors that live inside larger buffers (e.g. [B, N, H, d] "BSHD"
 * activations, or a fused QKV projection output):
 *
 *   q_strides, k_strides, v_strides, o_strides
 *            int64[3] in ELEMENTS: the distance between consecutive batches,
 *            heads and rows (query/key positions) of that tensor; the head dim
 *            is always contiguous.  NULL = the contiguous [B, heads, N, d]
 *            layout of fa_fwd.  Each value must be >= 0, the row stride >= d;
 *            q/k/v strides a multiple of 8, o strides a multiple of 4 (else
 *            FA_ERR_ALIGN).  Zero batch/head strides may broadcast q/k/v; O
 *            rows of different (b, h, row) must not overlap (else the result is
 *            unspecified).
 *   o        written in o_dtype: FA_DTYPE_F32, FA_DTYPE_F16 or FA_DTYPE_BF16
 *            (O is formed in fp32, divided by the row sum, then rounded to
 *            nearest even).
 *   lse      always fp32, contiguous [B, H, Nq].
 *
 * The keys of one (b, K/V head) are addressed with 32-bit byte offsets:
 * (Nk + 64) * row_stride * 2 must stay below 2^31 for K and V (else
 * FA_ERR_SHAPE).  Everything else as for fa_fwd_gqa.
 */
int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int H_kv, int Nq, int Nk, int d, const int64_t *q_strides,
              const int64_t *k_strides, const int64_t *v_strides, const int64_t *o_strides,
              float scale, int causal, const int32_t *kv_lens, int dtype, int o_dtype,
              void *stream);

/*
 * Exact attention backward from the forward's saved log-sum-exp (gpu-inference
 * page, section 02: the probabilities are recomputed, not stored; the row
 * term D, dK/dV and dQ.  Here the dQ pass also forms D, then the dK/dV pass
 * runs).  With P the forward's masked
 * softmax probabilities and dout = dL/dO:
 *   delta[i] = D_i = dO_i . O_i
 *   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . v_j - D_i),
 *   dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j.
 *
 *   q, dout  [B, H, Nq, d] f16/bf16 (dtype), contiguous; 16-byte aligned
 *   k, v     [B, H_kv, Nk, d] same dtype (H a multiple of H_kv); 16-byte aligned
 *   o        [B, H, Nq, d] float32: the forward's O for these inputs; 16-byte aligned
 *   lse      [B, H, Nq] float32: the forward's LSE; 4-byte aligned
 *   dq       [B, H, Nq, d] float32 output; 16-byte aligned
 *   dk, dv   [B, H_kv, Nk, d] float32 outputs (summed over the query heads that
 *            share each K/V head); 16-byte aligned
 *   delta    [2, B, H, Nq] float32 caller-owned scratch, 4-byte aligned: the dQ
 *            pass writes delta[0] = D and delta[1] = LSE * log2(e) (-inf stays
 *            -inf), the dK/dV pass reads both
 *   d        8..128, a multiple of 8 (computed on the d = 64 or 128 tiles, the
 *            columns past d as zeros); other head dims: FA_ERR_UNSUPPORTED
 *   scale, causal, kv_lens: as for the forward that produced o and lse.
 *
 * Rows with no valid key get dQ = 0; keys no row sees get dK = dV = 0.  Every
 * output element is written by exactly one block (no atomics): results are
 * bitwise reproducible.  (max(Nq, Nk) + 64) * d * 2 must stay below 2^31.
 */
int fa_bwd(const void *q, const void *k, const void *v, const float *o, const void *dout,
           const float *lse, float *dq, float *dk, float *dv, float *delta, int B, int H,
           int H_kv, int Nq, int Nk, int d, float scale, int causal, const int32_t *kv_lens,
           int dtype, void *stream);

/*
 * Decode attention over a paged KV cache (query length 1).
 *
 *   q           [S, H, d] f16/bf16; 16-byte aligned
 *   k_pages,
 *   v_pages     [num_pages, H, page_size, d] pools, same dtype; 16-byte aligned.
 *               Token t of sequence s lives in page page_table[s][t / page_size],
 *               row t % page_size.
 *   page_table  device int32 [S, max_pages_per_seq]; entries beyond a sequence's
 *               pages are ignored (their values are never used).  4-byte aligned
 *   kv_lens     device int32 [S]: number of cached tokens of each sequence, all of
 *               which the query attends to.  Clamped to [0, max_pages_per_seq *
 *               page_size].  A used table entry outside [0, num_pages) is clamped
 *               into range (result unspecified, no out-of-bounds access).
 *   o           [S, H, d] float32 output; 16-byte aligned
 *   lse         [S, H] float32 output; 4-byte aligned
 *   d           64 or 128;  page_size 16
 *   workspace   device buffer of at least
 *               fa_decode_workspace_bytes(S, H, d, max_pages_per_seq, page_size)
 *               bytes, 16-byte aligned, owned by the caller; its contents on
 *               entry do not matter.  NULL allowed only if that size is 0.
 *
 * A sequence with kv_len 0 gets O = 0 and LSE = -inf.  S or H of 0 is an empty
 * problem.  Long sequences are split into chunks of cached tokens whose
 * partial results are merged with the log-sum-exp rule; the split depends
 * only on logical token positions, so the result does not depend on where the
 * pages sit in the pool.
 */
int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                    const int32_t *page_table, const int32_t *kv_lens, float *o, float *lse,
                    int S, int H, int d, int page_size, int max_pages_per_seq, int num_pages,
                    float scale, int dtype, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * fa_decode_paged with grouped-query heads (see fa_fwd_gqa):
 *
 *   k_pages,
 *   v_pages     [num_pages, H_kv, page_size, d]; H a positive multiple of H_kv.
 *               Query head h reads K/V head h / (H / H_kv).
 *
 * The K/V rows of a page are read once for all the query heads that share
 * them.  Workspace: fa_decode_workspace_bytes(S, H, ...) with H the number of
 * QUERY heads.  Every other argument and error as for fa_decode_paged; H_kv < 1
 * or H not a multiple of H_kv (with H > 0) is FA_ERR_SHAPE.
 */
int fa_decode_paged_gqa(const void *q, const void *k_pages, const void *v_pages,
                        const int32_t *page_table, const int32_t *kv_lens, float *o, float *lse,
                        int S, int H, int H_kv, int d, int page_size, int max_pages_per_seq,
                        int num_pages, float scale, int dtype, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * fa_decode_paged_gqa without a workspace argument, for callers that cannot
 * allocate device memory at all (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The split-KV partials go to a
 * fixed scratch array inside the library instead: 40 MiB (41943040 bytes) of
 * device memory that every GPU the library runs on holds until the process
 * ends.  The call itself allocates and frees nothing.
 *
 *   Every argument, layout, alignment and error as for fa_decode_paged_gqa;
 *   the result is bitwise equal to that call's on the same inputs.
 *   FA_ERR_SCRATCH when fa_decode_workspace_bytes(S, H, d, max_pages_per_seq,
 *   page_size) exceeds 41943040 bytes (e.g. S = 32, H = 32, d = 128 fits with
 *   up to 624 pages of 16 tokens per sequence), checked before any HIP call.
 *
 * All calls on one GPU share that GPU's scratch: calls that overlap in time on
 * one GPU (other streams, other threads) race and give unspecified results;
 * serialise them (e.g. one stream).  The scratch's contents on entry do not
 * matter (nothing in it needs to start at zero).  The first call on each
 * device looks up the scratch's device address (hipGetSymbolAddress) with
 * that device current; a failure there is FA_ERR_HIP.
 */
int fa_decode_paged_noalloc(const void *q, const void *k_pages, const void *v_pages,
                            const int32_t *page_table, const int32_t *kv_lens, float *o,
                            float *lse, int S, int H, int H_kv, int d, int page_size,
                            int max_pages_per_seq, int num_pages, float scale, int dtype,
                            void *stream);

/*
 * Paged KV cache: append (inference kernel cookbook page, recipe 02 "KV Cache":
 * store each token's K and V once for every later decode step; recipe 03: in
 * fixed-size pages found through a page table).  Writes the K and V rows of
 * T new tokens -- a prefill chunk or one token per sequence at a decode step --
 * into the pools that fa_decode_paged reads:
 *
 *   k_new, v_new  [T, H_kv, d] f16/bf16, contiguous; 16-byte aligned
 *   seq_ids       device int32 [T]: the sequence of each token, in [0, S)
 *   positions     device int32 [T]: its logical position t in that sequence; the
 *                 rows go to page page_table[s][t / 16], row t % 16
 *   k_pages,
 *   v_pages       [num_pages, H_kv, page_size, d] pools (written); 16-byte aligned
 *   page_table    device int32 [S, max_pages_per_seq]
 *   d             a multiple of 8 from 8 to 256;  page_size 16
 *
 * A token whose seq id, position or page entry is out of range is skipped (no
 * write).  Two tokens with the same (sequence, position) in one call race.
 * T or S of 0 is an empty call.
 */
int fa_kv_append(const void *k_new, const void *v_new, const int32_t *seq_ids,
                 const int32_t *positions, int T, void *k_pages, void *v_pages,
                 const int32_t *page_table, int S, int H_kv, int d, int page_size,
                 int max_pages_per_seq, int num_pages, int dtype, void *stream);

/*
 * Paged KV cache: host-side page allocator (inference kernel cookbook page,
 * recipe 03: pages instead of one contiguous buffer per sequence; NanoInfer
 * page, paged KV-cache allocator).  Owns a host page table [max_seqs,
 * max_pages_per_seq] (-1 where unused) and a free list of the pool's pages
 * (a stack: the most recently freed page is reused first).  Pages are 16
 * tokens.  This object lives in HOST memory allocated by the library; it
 * touches no device memory: copy the table to the device array the kernels
 * read.  Calls on one pager are serialised internally.
 *
 *   fa_pager_create    NULL for sizes < 1 or too large, or host allocation failure
 *   fa_pager_reserve   grow sequence seq to hold len tokens (pages appended from
 *                      the free list; never shrinks).  FA_ERR_NOMEM when the free
 *                      list is too short (nothing changes), FA_ERR_SHAPE for a bad
 *                      seq or len > max_pages_per_seq * 16
 *   fa_pager_release   all pages of seq back to the free list; its length is 0
 *   fa_pager_length    tokens reserved for seq (-1 for a bad pager or seq)
 *   fa_pager_free_pages  pages on the free list (-1 for a NULL pager)
 *   fa_pager_copy_table  copy the table (max_seqs * max_pages_per_seq int32)
 *                      into dst; FA_ERR_SHAPE if dst_entries is smaller
 */
typedef struct fa_pager fa_pager;
fa_pager *fa_pager_create(int num_pages, int max_seqs, int max_pages_per_seq);
void fa_pager_destroy(fa_pager *p);
int fa_pager_reserve(fa_pager *p, int seq, int len);
int fa_pager_release(fa_pager *p, int seq);
int fa_pager_length(const fa_pager *p, int seq);
int fa_pager_free_pages(const fa_pager *p);
int fa_pager_copy_table(const fa_pager *p, int32_t *dst, size_t dst_entries);

/*
 * Pre-LayerNorm attention block: the encoder layer of the
 * Kernel-Inference-Engine page's charts (x -> LayerNorm -> dense Q/K/V ->
 * softmax(QK^T/sqrt(d)) V -> dense W_O -> + x), with the LayerNorm folded into
 * the Q/K/V projection so that no normalised activation is stored (the page's
 * fused kernel folds it into the attention prologue; its LayerNorm kernel uses
 * Welford's one-pass mean and variance).
 *
 * Matrices are row-major, contiguous, in the 16-bit dtype (FA_DTYPE_F16 or
 * FA_DTYPE_BF16), 16-byte aligned; dense weights are output-major [N, K] (row
 * n holds the K input weights of output n).  LayerNorm parameters, biases and
 * statistics are fp32, 16-byte aligned.  LayerNorm(x) = (x - mean) / sqrt(var
 * + eps) * gamma + beta with the row's population variance; eps must be finite
 * and >= 0 (else FA_ERR_ARG).
 *
 *   fa_ln_stats         mean[t] and rstd[t] = 1/sqrt(var + eps) of the T rows of
 *                       x [T, C] (C a multiple of 8).
 *   fa_ln_fold_weights  once per weight set: w_folded[n, k] = gamma[k] w[n, k]
 *                       rounded to the dtype, bias_folded[n] = bias[n] +
 *                       sum_k beta[k] w[n, k] (bias may be NULL = 0), colsum[n] =
 *                       sum_k w_folded[n, k].  w [N, C], C a multiple of 8.
 *   fa_ln_linear        y = LayerNorm(x) w^T + bias for x [T, C], from the
 *                       statistics and the folded weights: y[t, n] = rstd[t] *
 *                       (sum_k x[t, k] w_folded[n, k] - mean[t] colsum[n]) +
 *                       bias_folded[n], accumulated in fp32, rounded once to the
 *                       dtype.  y [T, N]; C a multiple of 64, N of 8.
 *   fa_linear           y = a w^T + bias (+ residual) for a [M, K], w [N, K],
 *                       bias [N] (NULL = 0), residual [M, N] (NULL = none); fp32
 *                       accumulation, one rounding.  K a multiple of 64, N of 8.
 *
 * Sizes: T, M of 0 is an empty call; negative sizes or K * 512 >= 2^31 are
 * FA_ERR_SHAPE; a C, K or N that is not the stated multiple is
 * FA_ERR_UNSUPPORTED.  Outputs must not overlap inputs.
 */
int fa_ln_stats(const void *x, float *mean, float *rstd, int T, int C, float eps, int dtype, void *stream);
int fa_ln_fold_weights(const float *gamma, const float *beta, const void *w, const float *bias,
                       void *w_folded, float *bias_folded, float *colsum, int N, int C, int dtype,
                       void *stream);
int fa_ln_linear(const void *x, const float *mean, const float *rstd, const void *w_folded,
                 const float *bias_folded, const float *colsum, void *y, int T, int C, int N,
                 int dtype, void *stream);
int fa_linear(const void *a, const void *w, const float *bias, const void *residual, void *y, int M,
              int K, int N, int dtype, void *stream);

/*
 * The whole block, y = x + Attention(LayerNorm(x) W_qkv^T + b_qkv) W_o^T + b_o,
 * for x [B*N, C] (token t = b*N + n), C = H*d:
 *
 *   w_qkv_folded, b_qkv_folded, colsum_qkv
 *                 fa_ln_fold_weights of W_qkv [(H + 2*H_kv)*d, C] (output rows:
 *                 the H query heads, then the H_kv key heads, then the H_kv
 *                 value heads, d each), b_qkv, gamma and beta
 *   w_o, b_o      W_o [C, H*d], b_o [C] (NULL = 0)
 *   y             [B*N, C] (must not overlap x)
 *   scale, causal, kv_lens   as for fa_fwd (kv_lens [B] or NULL)
 *   workspace     device memory of fa_prenorm_attention_workspace_bytes(B, N, H,
 *                 H_kv, d) bytes, 256-byte aligned, holding the stages in this
 *                 order, each starting on a 256-byte boundary: mean [B*N] and
 *                 rstd [B*N] fp32, qkv [B*N, (H + 2*H_kv)*d] and o [B*N, H*d] in
 *                 the dtype, lse [B, H, N] fp32 (readable after the call).
 *
 * Runs fa_ln_stats, fa_ln_linear (qkv), the attention forward on qkv in place
 * (fa_fwd_ex strides, o in the dtype), and fa_linear with x as the residual.
 * d as for fa_fwd_ex; C a multiple of 64; eps, scale, causal as above;
 * FA_ERR_WORKSPACE for a NULL or short workspace.
 */
size_t fa_prenorm_attention_workspace_bytes(int B, int N, int H, int H_kv, int d);
int fa_prenorm_attention(const void *x, const void *w_qkv_folded, const float *b_qkv_folded,
                         const float *colsum_qkv, const void *w_o, const float *b_o, void *y, int B,
                         int N, int H, int H_kv, int d, float eps, float scale, int causal,
                         const int32_t *kv_lens, int dtype, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Workspace bytes fa_decode_paged needs for these sizes (0 for invalid sizes). */
size_t fa_decode_workspace_bytes(int S, int H, int d, int max_pages_per_seq, int page_size);

/* Static, human-readable text for a status code. */
const char *fa_status_str(int status);

/* The hipError_t of this thread's most recent FA_ERR_HIP (0 if none). */
int fa_last_hip_error(void);

/* Library version, for the binding's sanity check. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
