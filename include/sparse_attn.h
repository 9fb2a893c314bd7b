/*
 * sparse_attn.h -- C ABI of the indexer-selected sparse attention library for AMD
 * Instinct MI355X (gfx950).  Library: libsparse_attn.so.
 *
 * The method (two stages):
 *   1. a lightweight indexer scores every preceding token,
 *        I(t,s) = sum_j w(t,j) * ReLU( q(t,j) . k(s) ),
 *      over H_I low-dimensional index heads (width d_I) and one index key k(s) per token
 *      -- "Sparse Attention and RL Optimization: Three Technical Breakthroughs in LLM
 *      Post-Training", section 2.2;
 *   2. each query keeps the top-k preceding tokens by that score and runs causal softmax
 *      attention over only those KV rows -- the same page, section 2.3 and the section
 *      2.5 pseudocode; "Long-Context LLMs Explained: Sparse Attention, Stable
 *      Reinforcement Learning, and Verifiable Synthetic Data", sections 2.2-2.4 (decode
 *      reads only the selected k KV entries of a paged cache, section 2.3; prefill and
 *      decode are tuned as separate phases, section 2.5).
 *
 * Conventions for every call below
 *   - Tensors are DEVICE pointers to caller-owned, contiguous, row-major memory, 16-byte
 *     aligned.  The library never frees or retains them after the call returns.
 *   - Element type of q, k, v, q_idx, k_idx is the handle's dtype (fp32 or bf16, given as
 *     raw bits).  w, scores, out and lse are always fp32; indices are int32.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and do
 *     not synchronise, allocate device memory or touch the host after launch.  Scratch
 *     memory is the caller's `ws` workspace, sized by sparse_attn_workspace_size().
 *   - Host-side validation happens before any launch; on failure nothing is launched and
 *     the status plus sparse_attn_last_error() explain why.  Values that live in device
 *     memory (indices, block tables, context lengths, per-sequence k) are range-checked
 *     by the kernels: offending entries are skipped (never dereferenced) and a bit is set
 *     in the handle's device error word, read back by sparse_attn_check().
 *   - Causality: query t sees keys s <= t (itself included); a decode query with context
 *     length n sees s < n, its own key being the last cached token.
 *   - Ties in top-k go to the lower token index.  With fewer than k visible tokens all
 *     visible tokens are selected and the remaining slots are -1.  Index lists are
 *     written in ascending token order.
 *   - A handle is not thread-safe; use one handle per host thread / stream.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sa_handle_s *sa_handle_t;

typedef enum {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = 1,  /* bad pointer, shape, size or config                    */
    SA_ERR_UNSUPPORTED = 2,  /* valid request this build does not serve               */
    SA_ERR_WORKSPACE = 3,    /* ws is NULL or smaller than sparse_attn_workspace_size */
    SA_ERR_HIP = 4,          /* a HIP runtime call failed (launch, copy, alloc)       */
    SA_ERR_DEVICE_CHECK = 5  /* sparse_attn_check(): a kernel flagged bad device data */
} sa_status_t;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype_t;

/* Bits of the device error word (sparse_attn_check). */
#define SA_DEVERR_INDEX_RANGE   1u  /* an attention index was >= the visible length    */
#define SA_DEVERR_BLOCK_TABLE   2u  /* a visible token's page was -1 or >= n_pages       */
#define SA_DEVERR_CTX_LEN       4u  /* ctx_len[b] outside [1, max_ctx]                   */
#define SA_DEVERR_TOPK          8u  /* topk[b] outside [1, max_topk]                     */
#define SA_DEVERR_ROW          16u  /* row_seq[t] / row_pos[t] out of range (row skipped) */
#define SA_DEVERR_SYNC         32u  /* acceptance_rate: a token's workgroups never met (alpha invalid) */

typedef struct {
    int32_t n_idx_heads;   /* H_I: index heads (e.g. 64)                                  */
    int32_t d_idx;         /* d_I: index head width (e.g. 128)                            */
    int32_t n_heads;       /* H: attention query heads (e.g. 16)                          */
    int32_t n_kv_heads;    /* H_kv: 1 (all heads share one KV row) or H                   */
    int32_t d_qk;          /* query/key width per head (e.g. 576)                         */
    int32_t d_v;           /* value width per head (e.g. 512)                             */
    int32_t v_from_k;      /* 1: the value is the first d_v columns of the key row (one
                              shared latent row per token, multi-head latent attention as
                              kept by the model in "A Guide to Sparse Attention and
                              Efficient Reinforcement Learning in LLM Long-Context
                              Inference", section 1); 0: separate v tensor             */
    int32_t page_size;     /* tokens per KV page for decode (e.g. 64)                     */
    int32_t max_topk;      /* largest k any call may ask for, 1..8192                      */
    sa_dtype_t dtype;      /* element type of q, k, v, q_idx, k_idx                       */
    float softmax_scale;   /* attention logit scale; 0 means 1/sqrt(d_qk)                 */
} sa_config_t;

/* Operations for sparse_attn_workspace_size(). */
#define SA_OP_PREFILL 1  /* n = L (sequence length), max_ctx ignored                    */
#define SA_OP_DECODE  2  /* n = B (batch), max_ctx = upper bound of every ctx_len[b]     */
#define SA_OP_TOPK    3  /* n = rows, max_ctx = cols                                      */
#define SA_OP_PROJECT 4  /* n = L rows of indexer_project_q, max_ctx ignored              */
#define SA_OP_PREFILL_BLOCKS 5  /* sparse_attn_prefill_blocks: n = L, max_ctx ignored     */
#define SA_OP_DECODE_BLOCKS  6  /* sparse_attn_decode_blocks: as SA_OP_DECODE             */
#define SA_OP_PREFILL_PAGED  7  /* sparse_attn_prefill_paged: n = T query rows, max_ctx   */
#define SA_OP_PREFILL_CHUNK  8  /* sparse_attn_prefill_chunk: n = C rows, max_ctx = pos0 + C */
#define SA_OP_PREFILL_VARLEN 9  /* sparse_attn_prefill_varlen: n = T rows, max_ctx           */
#define SA_OP_ACCEPT        10  /* acceptance_rate: n = T tokens, max_ctx = V (0: two-pass only) */

/* Create a handle for one configuration.  Validates the config, allocates the 4-byte
 * device error word on the current device (the only device allocation the library makes)
 * and picks kernels.  Returns SA_ERR_INVALID_ARG for an inconsistent config. */
sa_status_t sparse_attn_create(const sa_config_t *cfg, sa_handle_t *out);

/* A handle for host-side planning, on a machine with or without a GPU: the same configuration checks as
 * sparse_attn_create, workspace sizes for a device of n_cu compute units (1 .. 65535; the fused prefill's
 * candidate lists scale with it), and every call's host-side validation -- but no device is touched:
 * a call whose arguments pass validation returns SA_ERR_UNSUPPORTED instead of launching (and so does
 * sparse_attn_check).  For schedulers that size workspaces ahead of time, and for testing the argument
 * checks where no GPU is present.  Release it with sparse_attn_destroy. */
sa_status_t sparse_attn_create_host(const sa_config_t *cfg, int32_t n_cu, sa_handle_t *out);

/* Release a handle (synchronises the device before freeing the error word). */
void sparse_attn_destroy(sa_handle_t h);

/* Text of the last error on this handle ("" if none); with h == NULL, the last error of
 * sparse_attn_create on this thread.  Owned by the library, valid until the next call. */
const char *sparse_attn_last_error(sa_handle_t h);

/* Bytes of workspace a call of `op` at size n / max_ctx needs (may be 0). */
sa_status_t sparse_attn_workspace_size(sa_handle_t h, int op, int64_t n, int64_t max_ctx,
                                       size_t *bytes);

/* Synchronise `stream`, read and clear the device error word.  SA_OK if it was zero,
 * otherwise SA_ERR_DEVICE_CHECK with the bits in *bits (if bits != NULL). */
sa_status_t sparse_attn_check(sa_handle_t h, void *stream, uint32_t *bits);

/* Indexer scores of a whole sequence, materialised -- "Sparse Attention and RL
 * Optimization...", section 2.2 (formula) with the causal mask of the section 2.5
 * pseudocode.  A parity/debug entry: the [L, L] matrix is only built for L <= 16384.
 *   q_idx  [L, H_I, d_I]  dtype      index queries q(t,j)
 *   w      [L, H_I]       fp32       head weights w(t,j) (any sign)
 *   k_idx  [L, d_I]       dtype      index keys k(s), shared by all heads
 *   scores [L, L]         fp32 out   scores[t,s] = I(t,s) for s <= t, -inf for s > t
 * Errors: SA_ERR_INVALID_ARG (NULL pointer, L < 1), SA_ERR_UNSUPPORTED (L > 16384). */
sa_status_t indexer_scores(sa_handle_t h, const void *q_idx, const float *w, const void *k_idx,
                           int64_t L, float *scores, void *stream);

/* Per-row top-k of a score matrix -- "Sparse Attention and RL Optimization...", section
 * 2.3 (top-k preceding tokens per query by index score) and the `topk` step of the
 * section 2.5 pseudocode.
 *   scores    [rows, ld] fp32   row r's candidates are scores[r, 0 .. valid(r))
 *   valid_len [rows] int32 or NULL: valid(r) = valid_len[r] (must be in [1, cols]); NULL
 *             means the causal rule valid(r) = min(r + 1, cols)
 *   k_per_row [rows] int32 or NULL: k(r) = k_per_row[r] (1 <= k(r) <= k); NULL means k
 *   k         width of each idx row, 1 <= k <= max_topk
 *   idx       [rows, k] int32 out: the min(k(r), valid(r)) columns with the largest
 *             scores (ties -> lower column), ascending, then -1 padding
 * Scores must not be NaN.  ws may be NULL (the call needs no workspace).
 * Errors: SA_ERR_INVALID_ARG for NULL tensors, rows/cols < 1, ld < cols, k outside
 * [1, max_topk]; device-side SA_DEVERR_TOPK for bad valid_len / k_per_row entries. */
sa_status_t topk_select(sa_handle_t h, const float *scores, int64_t rows, int64_t cols, int64_t ld,
                        const int32_t *valid_len, const int32_t *k_per_row, int32_t k,
                        int32_t *idx, void *stream);

/* Two-tier (block -> token) selection of a score matrix -- "A Guide to Sparse Attention and
 * Efficient Reinforcement Learning in LLM Long-Context Inference", section 1.1 (fine-grained
 * token selection: the history is cut into fixed-size blocks, a few high-value blocks are kept
 * by their indexer scores, and token-level selection runs inside the kept blocks only).  Row r
 * (candidates scores[r, 0 .. valid(r)), valid and k(r) as in topk_select):
 *   1. block j is the tokens s < valid(r) with s / block_size == j (the last may be short);
 *      its score is the largest score among them;
 *   2. the first min(n_blocks, blocks) blocks by (block score desc, block index asc) are kept;
 *   3. idx row r gets the min(k(r), tokens in the kept blocks) tokens of the kept blocks with
 *      the largest scores (ties -> lower index), ascending, then -1 padding to width k.
 * With n_blocks >= k the result equals topk_select's.
 *   block_size  a power of two in [1, 1024]
 *   n_blocks    1 <= n_blocks <= 2048, n_blocks * block_size <= 16384
 * Scores must not be NaN.  Needs no workspace.
 * Errors: those of topk_select; SA_ERR_INVALID_ARG for block_size / n_blocks out of range;
 * SA_ERR_UNSUPPORTED if n_blocks * block_size > 16384 or cols / block_size > 16384. */
sa_status_t topk_select_blocks(sa_handle_t h, const float *scores, int64_t rows, int64_t cols, int64_t ld,
                               const int32_t *valid_len, const int32_t *k_per_row, int32_t k,
                               int32_t block_size, int32_t n_blocks, int32_t *idx, void *stream);

/* Causal prefill of one sequence: indexer -> per-query top-k -> attention over the
 * selected rows -- the whole pipeline of "Sparse Attention and RL Optimization...",
 * section 2.5 and "Long-Context LLMs Explained...", section 2.4.  Scores are produced
 * and consumed per block of queries in the workspace; the [L, L] matrix is never formed.
 *   q      [L, H, d_qk]     dtype    attention queries
 *   k      [L, H_kv, d_qk]  dtype    keys (the shared latent row when H_kv = 1)
 *   v      [L, H_kv, d_v]   dtype    values, or NULL when v_from_k = 1
 *   q_idx  [L, H_I, d_I], w [L, H_I] fp32, k_idx [L, d_I]: the indexer inputs
 *   topk   k, 1 <= k <= max_topk
 *   out    [L, H, d_v] fp32 out: softmax(scale q k_sel^T) v_sel per query and head
 *   lse    [L, H] fp32 out or NULL: log-sum-exp of the scaled logits (natural log)
 *   idx_out [L, topk] int32 out or NULL: the selected tokens (ascending, -1 padded)
 *   ws, ws_bytes: workspace of at least sparse_attn_workspace_size(SA_OP_PREFILL, L)
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_WORKSPACE, SA_ERR_HIP. */
sa_status_t sparse_attn_prefill(sa_handle_t h, const void *q, const void *k, const void *v,
                                const void *q_idx, const float *w, const void *k_idx, int64_t L,
                                int32_t topk, float *out, float *lse, int32_t *idx_out,
                                void *ws, size_t ws_bytes, void *stream);

/* sparse_attn_prefill with the two-tier selection of topk_select_blocks in place of the
 * per-query top-k ("A Guide to Sparse Attention and Efficient Reinforcement Learning in LLM
 * Long-Context Inference", section 1.1); every other argument as in sparse_attn_prefill.  The
 * scores of each block of query rows are materialised in the workspace, which must hold at
 * least sparse_attn_workspace_size(SA_OP_PREFILL_BLOCKS, L) bytes.  A row attends to fewer than
 * min(topk, t + 1) tokens when the kept blocks hold fewer; its idx_out row is -1 padded.
 * Errors: those of sparse_attn_prefill and topk_select_blocks (with cols = L). */
sa_status_t sparse_attn_prefill_blocks(sa_handle_t h, const void *q, const void *k, const void *v,
                                       const void *q_idx, const float *w, const void *k_idx, int64_t L,
                                       int32_t topk, int32_t block_size, int32_t n_blocks, float *out,
                                       float *lse, int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

/* One decode step for B sequences against paged caches -- "Long-Context LLMs
 * Explained...", section 2.3: the indexer scores the whole cached context, and attention
 * reads only the selected KV rows, located through the block table.
 *   q          [B, H, d_qk]           dtype   the new token's queries
 *   q_idx      [B, H_I, d_I], w [B, H_I] fp32: its indexer inputs
 *   kv_pages   [n_pages, page_size, H_kv, d_qk] dtype   key (latent) page pool
 *   v_pages    [n_pages, page_size, H_kv, d_v]  dtype   value pool, or NULL if v_from_k
 *   kidx_pages [n_pages, page_size, d_I]        dtype   index-key page pool
 *   block_table [B, max_blocks] int32: logical page j of sequence b is pool page
 *               block_table[b, j]; token s is slot s % page_size of page s / page_size
 *   ctx_len    [B] int32: n_b visible tokens (1 <= n_b <= max_ctx), the new token last
 *   topk       [B] int32: k_b (1 <= k_b <= max_topk); min(k_b, n_b) rows are attended
 *   max_ctx    host-side upper bound of every ctx_len (sizes the launch), <= max_blocks *
 *              page_size
 *   out [B, H, d_v] fp32 out; lse [B, H] fp32 out or NULL; idx_out [B, max_topk] int32 out
 *   or NULL (logical token positions, ascending, -1 padded)
 *   ws, ws_bytes: at least sparse_attn_workspace_size(SA_OP_DECODE, B, max_ctx)
 * Errors: SA_ERR_INVALID_ARG, SA_ERR_WORKSPACE, SA_ERR_HIP; device-side SA_DEVERR_* bits
 * for out-of-range ctx_len, topk or block-table entries (those sequences are skipped). */
sa_status_t sparse_attn_decode(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                               const void *kv_pages, const void *v_pages, const void *kidx_pages,
                               int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                               const int32_t *ctx_len, const int32_t *topk, int32_t B,
                               int32_t max_ctx, float *out, float *lse, int32_t *idx_out,
                               void *ws, size_t ws_bytes, void *stream);

/* sparse_attn_decode with the two-tier selection of topk_select_blocks in place of the
 * per-sequence top-k ("A Guide to Sparse Attention and Efficient Reinforcement Learning in LLM
 * Long-Context Inference", section 1.1): blocks are aligned to logical token 0, so with
 * block_size = page_size a block is one page of the sequence.  Every other argument as in
 * sparse_attn_decode; the workspace is sparse_attn_workspace_size(SA_OP_DECODE_BLOCKS, B,
 * max_ctx) bytes.  Errors: those of sparse_attn_decode and topk_select_blocks (with
 * cols = max_ctx). */
sa_status_t sparse_attn_decode_blocks(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                      const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                      const int32_t *ctx_len, const int32_t *topk, int32_t B,
                                      int32_t max_ctx, int32_t block_size, int32_t n_blocks, float *out,
                                      float *lse, int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

/* sparse_attn_decode for callers that cannot allocate device memory or size a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results and
 * device-side checks as sparse_attn_decode, without ws / ws_bytes: its scratch (scores, histograms,
 * indices, split-attention partials) is a device array of 64 MiB that the library holds on every device
 * it runs on until the process ends; its address is looked up once per device in sparse_attn_create.
 * The call allocates nothing and calls no allocating routine.  All calls on one device share that array
 * and each leaves it holding its own state: calls that overlap on one device (several streams or host
 * threads at once) race and give undefined results; serialise them.
 * Errors: those of sparse_attn_decode; SA_ERR_UNSUPPORTED when the step needs more than the array holds
 * (sparse_attn_workspace_size(SA_OP_DECODE, B, max_ctx) > 64 MiB; B = 64 at max_ctx = 131072 with
 * max_topk = 2048 needs about 48 MB). */
sa_status_t sparse_attn_decode_noalloc(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                       const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                       int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                       const int32_t *ctx_len, const int32_t *topk, int32_t B, int32_t max_ctx,
                                       float *out, float *lse, int32_t *idx_out, void *stream);

/* Query rows against paged caches: chunked prefill (new tokens of a sequence whose earlier tokens
 * are already cached), varlen batches of several sequences, and several new tokens per sequence in
 * one decode step.  Query row t is the token at position p = row_pos[t] of sequence
 * b = row_seq[t]; it scores the tokens s <= p of that sequence in the paged index-key cache, keeps
 * its top-k, and attends to the selected rows of the paged KV cache -- "Long-Context LLMs
 * Explained...", section 2.3 (selection over a paged cache) with the causal look-back of "Sparse
 * Attention and RL Optimization...", section 2.5.  The caches must already hold every token
 * s <= p (write the new tokens' rows first, e.g. with indexer_project_k).
 *   q [T, H, d_qk], q_idx [T, H_I, d_I], w [T, H_I] fp32: the T query rows, in any order
 *   kv_pages, v_pages, kidx_pages, n_pages: the page pools of sparse_attn_decode
 *   block_table [n_seqs, max_blocks] int32 (host-known n_seqs, max_blocks)
 *   row_seq, row_pos [T] int32 (device): sequence in [0, n_seqs), position in [0, max_ctx)
 *   max_ctx    host-side bound of every row_pos + 1, <= max_blocks * page_size
 *   topk       k, 1 <= k <= max_topk; row t attends to min(k, p + 1) tokens
 *   out [T, H, d_v] fp32; lse [T, H] fp32 or NULL; idx_out [T, topk] int32 or NULL (positions,
 *   ascending, -1 padded)
 *   ws, ws_bytes: at least sparse_attn_workspace_size(SA_OP_PREFILL_PAGED, T, max_ctx)
 * With bf16, H_I = 64, d_I = 128, 64-token pages, T <= 16384 and max_ctx <= 524288 the rows are sorted by
 * (sequence, position) on the device and each sequence's rows run as tiles of 8 rows of the fused prefill
 * indexer / top-k, sharing every key tile (one page); otherwise each row is scored alone.  Both give the
 * same scores, term for term in the same order.
 * A row whose (row_seq, row_pos) is out of range sets SA_DEVERR_ROW and is skipped (its outputs
 * are unspecified).  Errors: SA_ERR_INVALID_ARG, SA_ERR_WORKSPACE, SA_ERR_HIP; device-side bits as
 * in sparse_attn_decode. */
sa_status_t sparse_attn_prefill_paged(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                      const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table, int32_t n_seqs,
                                      int32_t max_blocks, const int32_t *row_seq, const int32_t *row_pos,
                                      int64_t T, int32_t max_ctx, int32_t topk, float *out, float *lse,
                                      int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

/* Prefill of a batch of sequences against their paged caches (varlen layout): sequence b owns the
 * query rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1, which are its newest tokens, at positions
 * ctx_len[b] - n_new .. ctx_len[b] - 1 (n_new = cu_seqlens[b + 1] - cu_seqlens[b]); the caches must
 * already hold all ctx_len[b] tokens.  The same computation as sparse_attn_prefill_paged with those
 * (row_seq, row_pos) pairs -- "Sparse Attention and RL Optimization...", sections 2.2, 2.3 and 2.5
 * (the batched teacher-forcing pass); "Long-Context LLMs Explained...", section 2.3 -- for the case
 * where each sequence's rows are contiguous but the layout is known only on the device: with bf16,
 * H_I = 64, d_I = 128 and 64-token pages (and max_ctx <= 524288) every sequence's rows run as tiles of
 * 8 rows of the fused prefill indexer / top-k, sharing every key tile (one page) between them.
 *   q [T, H, d_qk], q_idx [T, H_I, d_I], w [T, H_I] fp32; pools and block_table [n_seqs, max_blocks]
 *   as in sparse_attn_decode
 *   cu_seqlens [n_seqs + 1] int32 (device): 0 = cu_seqlens[0] <= ... <= cu_seqlens[n_seqs] = T
 *   ctx_len [n_seqs] int32 (device): cached tokens per sequence, n_new <= ctx_len[b] <= max_ctx
 *   max_ctx    host-side bound of every ctx_len, <= max_blocks * page_size; topk in [1, max_topk]
 *   out [T, H, d_v] fp32; lse [T, H] or NULL; idx_out [T, topk] or NULL (positions, ascending, -1 pad)
 *   ws, ws_bytes: at least sparse_attn_workspace_size(SA_OP_PREFILL_VARLEN, T, max_ctx)
 * A sequence that breaks these bounds sets SA_DEVERR_ROW and its rows are skipped (a row of no valid
 * sequence gets -1 indices when the fused tiles run; its outputs are otherwise unspecified).  Errors:
 * SA_ERR_INVALID_ARG, SA_ERR_WORKSPACE, SA_ERR_HIP; device-side bits as in sparse_attn_decode. */
sa_status_t sparse_attn_prefill_varlen(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                       const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                       int64_t n_pages, const int32_t *block_table, int32_t n_seqs,
                                       int32_t max_blocks, const int32_t *cu_seqlens, const int32_t *ctx_len,
                                       int64_t T, int32_t max_ctx, int32_t topk, float *out, float *lse,
                                       int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

/* Chunked prefill of one sequence against its paged caches: query row i is the token at position
 * pos0 + i (i < C) of the sequence whose block-table row is block_table_row [max_blocks]; it sees the
 * tokens 0 .. pos0 + i, which the caches must already hold.  The same computation as
 * sparse_attn_prefill_paged with row_seq = 0, row_pos = pos0 + i, for the common case where the
 * chunk is known on the host: with bf16, H_I = 64, d_I = 128 and 64-token pages (and pos0 + C <=
 * 524288) the rows run as tiles of the fused prefill indexer / top-k, sharing every key tile (one
 * page) between 8 rows -- "Sparse Attention and RL Optimization...", sections 2.2, 2.3 and 2.5;
 * "Long-Context LLMs Explained...", section 2.3.
 *   q [C, H, d_qk], q_idx [C, H_I, d_I], w [C, H_I] fp32; pools as in sparse_attn_decode
 *   pos0 >= 0, C >= 1, pos0 + C <= max_blocks * page_size; topk in [1, max_topk]
 *   out [C, H, d_v] fp32; lse [C, H] or NULL; idx_out [C, topk] or NULL (positions, ascending, -1 pad)
 *   ws, ws_bytes: at least sparse_attn_workspace_size(SA_OP_PREFILL_CHUNK, C, pos0 + C)
 * A block-table entry of a visible page outside [0, n_pages) sets SA_DEVERR_BLOCK_TABLE; its tokens are
 * given no weight.  Errors: SA_ERR_INVALID_ARG, SA_ERR_WORKSPACE, SA_ERR_HIP. */
sa_status_t sparse_attn_prefill_chunk(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                      const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table_row, int32_t max_blocks,
                                      int64_t pos0, int64_t C, int32_t topk, float *out, float *lse,
                                      int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

/* Index-space projections -- the first lines of the "Sparse Attention and RL Optimization...",
 * section 2.5 pseudocode: the index query and key are linear maps of the attention query and
 * key (i_q = W_iq(q), i_k = W_ik(k)); the head weights w(t, j) of the section 2.2 score are one
 * more linear map of the query.  bf16 handles only (SA_ERR_UNSUPPORTED otherwise).  Weights are
 * row-major [out, in] bf16; accumulation is fp32; bf16 outputs are rounded to nearest even.
 *
 * indexer_project_q, for each of the L query rows q[t] (H * d_qk values, [L, H, d_qk]):
 *   q_idx[t] = W_iq q[t]   W_iq [H_I * d_I, H * d_qk]  ->  q_idx [L, H_I, d_I] bf16
 *   w[t]     = W_w  q[t]   W_w  [H_I, H * d_qk]        ->  w [L, H_I] fp32
 *   Either pair (W_iq, q_idx) or (W_w, w) may be NULL to skip it.  One kernel computes both in a
 *   single pass over q: [W_iq; W_w] is the second operand of one tiled bf16 MFMA GEMM (fp32
 *   accumulation), whose last column tile is W_w's.  Needs H * d_qk a multiple of 64, H_I * d_I a
 *   multiple of 256 and H_I <= 256.  Needs no workspace: ws and ws_bytes are ignored (may be NULL / 0;
 *   sparse_attn_workspace_size(SA_OP_PROJECT, L) is 0).
 * Errors: SA_ERR_INVALID_ARG (NULL q, L < 1, both pairs NULL, a pair half NULL, misaligned),
 * SA_ERR_UNSUPPORTED (not bf16, or another shape), SA_ERR_HIP. */
sa_status_t indexer_project_q(sa_handle_t h, const void *q, int64_t L, const void *W_iq, const void *W_w,
                              void *q_idx, float *w, void *ws, size_t ws_bytes, void *stream);

/* indexer_project_k: k_idx[t] = W_ik k[t] for the L key rows k[t] (the H_kv * d_qk key row:
 * the latent row when H_kv = 1), W_ik [d_I, H_kv * d_qk] bf16, bf16 out.  Needs d_I = 128 and
 * a key row H_kv * d_qk of 128, 256, 512 or 576 elements (W_ik is held in LDS).
 *   block_table == NULL: k_idx is [L, d_I], row t = token t.
 *   block_table != NULL ([n_seqs, max_blocks] int32): k_idx is the paged index-key pool
 *   [n_pages, page_size, d_I] of sparse_attn_decode, and row t is the token at position
 *   p = row_pos[t] (or pos0 + t when row_pos is NULL) of sequence b = row_seq[t] (or 0 when
 *   row_seq is NULL): it goes to page block_table[b * max_blocks + p / page_size], slot
 *   p % page_size.  A prefill of one sequence
 *   passes row_seq = row_pos = NULL and its first position pos0; a decode step passes one row
 *   per sequence with row_seq[t] = t and row_pos[t] = ctx_len[t] - 1.  A row whose page entry
 *   is outside [0, n_pages) (or whose sequence is outside [0, n_seqs), or whose position is
 *   negative or beyond max_blocks pages) is not written and sets SA_DEVERR_BLOCK_TABLE.
 * Needs no workspace.  Errors: SA_ERR_INVALID_ARG (NULL k / W_ik / k_idx, L < 1, misaligned,
 * n_seqs, max_blocks or n_pages < 1 with a block table), SA_ERR_UNSUPPORTED (not bf16,
 * d_I != 128, another key-row width). */
sa_status_t indexer_project_k(sa_handle_t h, const void *k, int64_t L, const void *W_ik, void *k_idx,
                              const int32_t *block_table, int32_t n_seqs, int32_t max_blocks, int64_t n_pages,
                              const int32_t *row_seq, const int32_t *row_pos, int64_t pos0, void *stream);

/* Per-token acceptance rate between a dense and a sparse next-token distribution -- "Sparrow:
 * Sparse Rollout for Stable and Efficient Long-context RL of Large Language Models", section 3.1:
 * alpha(t) = E_{x~q}[min(p(x)/q(x), 1)] = sum_x min(p(x), q(x)), where p and q are the softmax of
 * logit rows t of logits_p and logits_q over the vocabulary.
 *   logits_p, logits_q [T, ld] fp32 (row t: entries 0 .. V-1); each row needs a finite entry
 *   alpha [T] fp32 out, in [0, 1]
 *   ws, ws_bytes: NULL / 0, or at least sparse_attn_workspace_size(SA_OP_ACCEPT, T, V) bytes
 * With a workspace (and V % 4 == 0, ld % 4 == 0, 16-byte aligned rows, V <= 450560 on 256 CUs) each
 * logit is read once: a token's rows are split over a group of co-resident workgroups that hold
 * them in registers and exchange their normalisers through the workspace; the launch takes every
 * CU until it ends, and a group whose members cannot all be scheduled together gives up after a
 * bounded wait with SA_DEVERR_SYNC.  Otherwise (no workspace, or a size of 0) both rows are
 * streamed twice (max and sum of exp, then the sum of minima).  fp32 arithmetic either way; the
 * result is deterministic for a given path.  Calls sharing one workspace must not overlap.
 * Errors: SA_ERR_INVALID_ARG (NULL pointer, T < 1, V < 1, ld < V), SA_ERR_WORKSPACE (ws given
 * but smaller than the size above). */
sa_status_t acceptance_rate(sa_handle_t h, const float *logits_p, const float *logits_q, int64_t T, int64_t V,
                            int64_t ld, float *alpha, void *ws, size_t ws_bytes, void *stream);

/* The lower-tail statistic of the acceptance rate per bin of positions -- the same page and
 * section (the 5-percentile of the per-token values in bins of 2K positions).  Token t falls in
 * bin pos[t] / bin_size; tokens with a negative position or a bin >= n_bins are ignored.  Per
 * bin j: count[j] tokens, mean[j] (NaN if empty) and pct[j] = x[lo] + (h - lo) (x[lo + 1] - x[lo])
 * with x the bin's values ascending, h = (count - 1) percentile / 100 and lo = floor(h) (the value
 * itself at the top rank; NaN if empty).
 *   alpha [T] fp32, pos [T] int32; count [n_bins] int32 out, mean, pct [n_bins] fp32 out
 * Needs no workspace.  Errors: SA_ERR_INVALID_ARG (NULL pointer, T < 1, bin_size < 1,
 * n_bins < 1, percentile outside [0, 100]). */
sa_status_t acceptance_bin_stats(sa_handle_t h, const float *alpha, const int32_t *pos, int64_t T,
                                 int32_t bin_size, int32_t n_bins, float percentile, int32_t *count,
                                 float *mean, float *pct, void *stream);

/* Kernel timing, a tracing aid for benchmarks.  While enabled, every kernel the handle
 * launches is bracketed by a pair of hipEvents recorded on the launch stream, and the
 * elapsed times are summed per kernel kind.  Enabling resets the sums; it creates events
 * (host-side runtime objects) but allocates no device memory in the library's own name.
 * sparse_attn_profile_read synchronises on the recorded events and returns, per kind, the
 * summed milliseconds and the number of launches (arrays of SA_KERNEL_COUNT entries).
 * While profiling is on, calls may synchronise the host when many events are pending. */
#define SA_KERNEL_INDEXER   0  /* indexer scores (prefill blocks, decode, indexer_scores) */
#define SA_KERNEL_TOPK      1  /* per-row top-k selection                                 */
#define SA_KERNEL_ATTENTION 2  /* attention over the selected rows                        */
#define SA_KERNEL_MERGE     3  /* merge of split decode attention states                  */
#define SA_KERNEL_PROJECT   4  /* index-space projections (indexer_project_q / _k)         */
#define SA_KERNEL_ACCEPT    5  /* acceptance rate and its per-bin statistics               */
#define SA_KERNEL_COUNT     6
sa_status_t sparse_attn_profile(sa_handle_t h, int enable);
sa_status_t sparse_attn_profile_read(sa_handle_t h, double *total_ms, int64_t *launches);

/* Device peaks measured on the box -- the denominators a benchmark reports beside the published ones.
 * Measurement aids only: nothing of the method runs in them.
 *
 * sparse_attn_peak_mfma: one workgroup of eight waves per compute unit (two per SIMD, the fused prefill
 * indexer's occupancy) runs `iters` iterations of eight v_mfma_f32_32x32x16_bf16 each (32768 flop per
 * MFMA, four independent fp32 accumulators), every MFMA on a different pair of A / B fragments taken from
 * `operands` (caller-filled random bf16, at least 1 MiB, 16-byte aligned), so the multipliers switch as
 * on real data.  Flop per launch = n_cu * 8 waves * iters * 8 * 32768.  clocks [256] uint64 (device):
 * for workgroups 0 .. min(n_cu, 64) - 1, four counters each -- shader-clock counter (s_memtime) before and
 * after the loop, then the 100 MHz reference counter (s_memrealtime) before and after -- from which the
 * clock the loop ran at follows.  sink: one float of device memory (written only to keep results live).
 *
 * sparse_attn_peak_stream: bytes (a positive multiple of 16) of src read once with 16-byte non-temporal
 * loads (dst == NULL; sink: one float of device memory) or copied to dst (sink may be NULL), by 8
 * workgroups of 256 threads per compute unit, grid-stride.
 *
 * Both are asynchronous on `stream`; time them with events.  Errors: SA_ERR_INVALID_ARG (NULL handle or
 * pointer, misaligned pointer, iters < 1, bad bytes, not the handle's device), SA_ERR_HIP. */
sa_status_t sparse_attn_peak_mfma(sa_handle_t h, const void *operands, int32_t iters, uint64_t *clocks,
                                  float *sink, void *stream);
sa_status_t sparse_attn_peak_stream(sa_handle_t h, const void *src, void *dst, int64_t bytes, float *sink,
                                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
