// Host-side internals of libsparse_attn: the handle and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <utility>
#include <vector>

#include "../../include/sparse_attn.h"

struct sa_handle_s {
    sa_config_t cfg;
    float scale;            // resolved attention logit scale
    uint32_t *d_err;        // device error word (SA_DEVERR_* bits)
    int device;
    int n_cu;               // compute units of the device (sizes persistent grids)
    bool fast_indexer;      // bf16, H_I = 64, d_I = 128: MFMA indexer kernels
    bool fast_decode;       // fast_indexer with 64-token pages: the paged decode kernels
    bool fast_attn;         // bf16, H = 16, H_kv = 1, d_qk = 576, d_v = 512, v_from_k
    std::string last_error;

    // kernel timing (sparse_attn_profile)
    bool profiling = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[SA_KERNEL_COUNT];
    std::vector<hipEvent_t> spare_events;
    double total_ms[SA_KERNEL_COUNT] = {};
    int64_t launches[SA_KERNEL_COUNT] = {};
};

namespace sa {

// Brackets one kernel launch with events while the handle is profiling.
class KernelTimer {
public:
    KernelTimer(sa_handle_s &h, int kind, hipStream_t st);
    ~KernelTimer();

private:
    sa_handle_s &h_;
    int kind_;
    hipStream_t st_;
    hipEvent_t start_ = nullptr;
};

// Synchronise on and account every pending event pair.
hipError_t drain_profile(sa_handle_s &h);

// Where the index keys / KV rows of a query row live.
//  contiguous: row s of sequence = base + s * row_elems
//  paged:      token s of sequence b = pool page block_table[b * max_blocks + s / page_size],
//              slot s % page_size; pages hold page_size rows of row_elems elements.  Query row r
//              belongs to sequence b = row_seq[r] (row_seq != nullptr, entries already checked),
//              else b = r.
struct RowSource {
    const void *base;
    int64_t row_elems;              // elements per token row
    const int32_t *block_table;     // nullptr -> contiguous
    int32_t max_blocks;
    int32_t page_size;
    int64_t n_pages;
    const int32_t *row_seq = nullptr;
    __device__ int64_t seq_of(int64_t r) const { return row_seq ? (int64_t)row_seq[r] : r; }
};

// Which keys a query row sees: keys s < visible(r), where visible(r) = causal_row0 + r + 1
// (prefill) or ctx_len[r] (decode; must lie in [1, max_ctx]).
struct Visibility {
    int64_t causal_row0;
    const int32_t *ctx_len;         // nullptr -> causal rule
    int32_t max_ctx;
};

// ---- indexer: scores[r, s] for s < n_cols; s >= visible(r) gets -inf -------------------
hipError_t launch_indexer(sa_handle_s &h, const void *q_idx, const float *w,
                          int64_t n_rows, RowSource keys, Visibility vis, float *scores,
                          int64_t ld, int64_t n_cols, hipStream_t st);

// ---- per-row top-k over materialised scores ----------------------------------------------
// valid(r) = valid_len ? valid_len[r] : min(causal_row0 + r + 1, cols); k(r) = k_per_row ?
// k_per_row[r] : k.  idx row r gets the min(k(r), valid(r)) best columns ascending, -1 pad.
hipError_t launch_topk(sa_handle_s &h, const float *scores, int64_t ld, int64_t rows, int64_t cols,
                       const int32_t *valid_len, int64_t causal_row0, const int32_t *k_per_row,
                       int32_t k, int32_t *idx, int64_t idx_ld, uint32_t *err, hipStream_t st);

// ---- two-tier (block -> token) selection over materialised scores ------------------------
// Rows as in launch_topk.  Blocks of block_size tokens (a power of two, <= 1024) are ranked by
// their best score, the first min(n_blocks, blocks) are kept, and the min(k(r), candidates)
// best tokens inside them are written ascending, -1 padded to idx_ld.  The host guarantees
// ceil(cols / block_size) <= kBlockSelectMaxItems, n_blocks <= kBlockSelectMaxKept and
// n_blocks * block_size <= kBlockSelectMaxItems (everything is held in LDS).  pmax (optional, only
// with block_size >= 64): row r's order keys of the largest score of each 64-token span of its
// valid tokens, stride pmax_ld; block maxima are then combined from it instead of the scores.
constexpr int kBlockSelectMaxItems = 16384;
constexpr int kBlockSelectMaxKept = 2048;
hipError_t launch_block_topk(sa_handle_s &h, const float *scores, int64_t ld, int64_t rows, int64_t cols,
                             const int32_t *valid_len, int64_t causal_row0, const int32_t *k_per_row, int32_t k,
                             int32_t block_size, int32_t n_blocks, const uint32_t *pmax, int64_t pmax_ld,
                             int32_t *idx, int64_t idx_ld, uint32_t *err, hipStream_t st);

// ---- attention over selected rows --------------------------------------------------------
// Query row r attends to the first m(r) = min(k(r), visible(r)) entries of idx row r.
struct Selection {
    const int32_t *idx;
    int64_t idx_ld;
    int32_t k;                      // k(r) = k_per_row ? k_per_row[r] : k
    const int32_t *k_per_row;
};

// Rows with a context-length array (decode) may split each row's selection over workgroups
// (allow_split; ws then holds attention_workspace(h, n_rows, true) bytes); otherwise one
// workgroup attends to each row.
hipError_t launch_attention(sa_handle_s &h, const void *q, int64_t n_rows,
                            RowSource kv, RowSource v, Visibility vis, Selection sel,
                            float *out, float *lse, void *ws, hipStream_t st, bool allow_split = true);

// ---- fused prefill indexer + streaming top-k (bf16, H_I = 64, d_I = 128) ---------------
// idx [L, topk] gets every row's selection; ws holds prefill_topk_workspace(h, L, pos0) bytes.
// Row i is the token at position pos0 + i; keys are the tokens 0 .. pos0 + L - 1: rows of k_idx, or
// (table != nullptr) 64-token pages of the pool k_idx [n_pages, 64, d_I], page j of the sequence
// being table[j] (table holds at most kPrefillMaxPages entries for the keys).
constexpr int64_t kPrefillMaxPages = 8192;
// With block_keys != nullptr the kernel selects nothing: every row with more than keys_above visible
// keys gets, in block_keys [L, prefill_block_keys_ld(L, pos0)] (row i, tile j), the order key of the best
// score among the keys it sees in 64-key tile j (for every tile it sees), and idx is not written.
size_t prefill_topk_workspace(const sa_handle_s &h, int64_t L, int64_t pos0 = 0);
size_t prefill_block_keys_ld(int64_t L, int64_t pos0);
hipError_t launch_prefill_topk(sa_handle_s &h, const void *q_idx, const float *w, const void *k_idx,
                               int64_t L, int32_t topk, int32_t *idx, void *ws, hipStream_t st,
                               const int32_t *table = nullptr, int64_t n_pages = 0, int64_t pos0 = 0,
                               uint32_t *block_keys = nullptr, int64_t keys_above = 0);
// A batch of sequences on the same row tiles: sequence b owns query rows cu[b] .. cu[b + 1] - 1, the newest
// of its ctx_len[b] cached tokens (64-token pages of kidx_pages, block-table row b of block_table with
// stride max_blocks); max_ctx <= kPrefillMaxPages * 64.  ws holds prefill_varlen_workspace(h, T, max_ctx)
// bytes.  launch_varlen_rows writes each row's sequence and position to row_seq / row_pos [T] ((-1, -1)
// and an empty selection in idx for a row of no valid sequence); it runs first.
size_t prefill_varlen_workspace(const sa_handle_s &h, int64_t T, int32_t max_ctx);

// Rows that each name their (sequence, position) -- sparse_attn_prefill_paged -- on the fused prefill row tiles:
// the rows are sorted by (sequence, position) on the device and each sequence's run is cut into tiles of 8 rows.
// Needs the fast decode shapes, T <= 16384 and max_ctx <= kPrefillMaxPages * 64.  Rows out of range set
// SA_DEVERR_ROW and get empty index lists.  ws holds prefill_rows_workspace(h, T, max_ctx).
bool prefill_rows_fused(const sa_handle_s &h, int64_t T, int32_t max_ctx);
size_t prefill_rows_workspace(const sa_handle_s &h, int64_t T, int32_t max_ctx);
hipError_t launch_prefill_rows(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                               int64_t n_pages, const int32_t *block_table, int32_t max_blocks, const int32_t *row_seq,
                               const int32_t *row_pos, int32_t n_seqs, int64_t T, int32_t max_ctx, int32_t topk,
                               int32_t *idx, void *ws, hipStream_t st);
hipError_t launch_varlen_rows(sa_handle_s &h, const int32_t *cu, const int32_t *ctx_len, int32_t n_seqs, int64_t T,
                              int32_t max_ctx, int32_t topk, int32_t *idx, int32_t *row_seq, int32_t *row_pos,
                              hipStream_t st);
hipError_t launch_prefill_varlen(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                                 int64_t n_pages, const int32_t *block_table, int32_t max_blocks, const int32_t *cu,
                                 const int32_t *ctx_len, int32_t n_seqs, int64_t T, int32_t max_ctx, int32_t topk,
                                 int32_t *idx, void *ws, hipStream_t st);

// ---- paged decode indexer + per-sequence top-k (bf16, H_I = 64, d_I = 128, 64-token pages) --
struct DecodeTopkLayout {
    int64_t ld;          // score row stride (floats)
    int64_t pmax_ld;     // page-maxima row stride (uint32 order keys, one per 64-token page)
    int64_t n_chunks;    // top-k workgroups per sequence (token chunks)
    // byte offsets in the workspace: scores, histograms, page maxima, the per-sequence candidate lists
    // (keys, indices), each chunk's (offset, count) in them, two sync words per sequence (list fill, arrivals)
    size_t scores, hist, pmax, cand_keys, cand_idx, chunk_info, sync, total;
};
DecodeTopkLayout decode_topk_layout(int64_t B, int64_t max_ctx);
// idx [B, max_topk] gets each sequence's selection; ws holds decode_topk_layout(B, max_ctx).total
hipError_t launch_decode_indexer_topk(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                      const int32_t *ctx_len, const int32_t *topk_b, int32_t B, int32_t max_ctx,
                                      int32_t *idx, void *ws, hipStream_t st);

// Two-tier prefill, second pass (bf16, H_I = 64, d_I = 128, block_size a multiple of 64): row i (position
// pos0 + i) keeps n_blocks blocks by the tile keys launch_prefill_topk wrote (rows with more than
// n_blocks * block_size visible keys), scores their tokens and writes its top-topk to idx [L, topk].
// Keys are rows of k_idx, or (table != nullptr) 64-token pages of the pool k_idx, page j being table[j].
hipError_t launch_block_rescore_topk(sa_handle_s &h, const void *q_idx, const float *w, const void *k_idx,
                                     const int32_t *table, int64_t n_pages, int64_t L, int64_t pos0, int32_t topk,
                                     int32_t block_size, int32_t n_blocks, const uint32_t *bkeys, int64_t bkeys_ld,
                                     int32_t *idx, hipStream_t st);

// The paged decode indexer alone: sequence b's scores land at ws + layout.scores, row stride
// layout.ld (floats), for tokens s < ctx_len[b]; with page_maxima, the order key of the largest
// score of each visible 64-token logical page lands at ws + layout.pmax, row stride layout.pmax_ld.
// Row b reads the block-table row row_seq[b] (row_seq != nullptr, entries already checked) or b.
hipError_t launch_decode_indexer(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                                 int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                 const int32_t *ctx_len, const int32_t *row_seq, int32_t B, int32_t max_ctx,
                                 bool page_maxima, void *ws, hipStream_t st);
// The per-row top-k over the scores and histograms launch_decode_indexer left in ws: row b keeps
// min(topk_b[b], ctx_len[b]) tokens (topk_b[b] <= max_topk), written to idx [B, max_topk].
hipError_t launch_decode_topk(sa_handle_s &h, const int32_t *ctx_len, const int32_t *topk_b, int32_t max_topk,
                              int32_t B, int32_t max_ctx, int32_t *idx, void *ws, hipStream_t st);

// ---- query rows against paged caches --------------------------------------------------
// Checks (row_seq[t], row_pos[t]) (sequence in [0, n_seqs), position in [0, max_ctx); a bad row
// sets SA_DEVERR_ROW) and writes seq[t] (0 for a bad row), ctx[t] = row_pos[t] + 1 (0 for a bad
// row, which every later kernel skips) and budget[t] = topk.
hipError_t launch_paged_rows(sa_handle_s &h, const int32_t *row_seq, const int32_t *row_pos, int64_t T,
                             int32_t n_seqs, int32_t max_ctx, int32_t topk, int32_t *seq, int32_t *ctx,
                             int32_t *budget, hipStream_t st);

// ---- acceptance rate between two next-token distributions ---------------------------------
// The single-read path's workgroups per token (0: V does not suit it) and its workspace (0 likewise).
int acceptance_group(const sa_handle_s &h, int64_t V);
size_t acceptance_workspace(const sa_handle_s &h, int64_t T, int64_t V);
// ws: acceptance_workspace(h, T, V) bytes for the single-read path, or nullptr for the two-pass kernel.
hipError_t launch_acceptance_rate(sa_handle_s &h, const float *lp, const float *lq, int64_t T, int64_t V, int64_t ld,
                                  float *alpha, void *ws, hipStream_t st);
hipError_t launch_bin_stats(sa_handle_s &h, const float *alpha, const int32_t *pos, int64_t T, int32_t bin_size,
                            int32_t n_bins, float percentile, int32_t *count, float *mean, float *pct, hipStream_t st);

// ---- index-space projections (bf16) ---------------------------------------------------
size_t projection_workspace();
sa_status_t launch_project_q(sa_handle_s &h, const void *q, int64_t L, const void *W_iq, const void *W_w,
                             void *q_idx, float *w, void *ws, size_t ws_bytes, hipStream_t st);
hipError_t launch_project_k(sa_handle_s &h, const void *k, int64_t L, const void *W_ik, void *k_idx,
                            const int32_t *block_table, int32_t n_seqs, int32_t max_blocks, int64_t n_pages,
                            const int32_t *row_seq, const int32_t *row_pos, int64_t pos0, hipStream_t st);
void destroy_projection_state(sa_handle_s &h);

// Workspace bytes launch_attention needs for n_rows decode rows (split partials).
size_t attention_workspace(const sa_handle_s &h, int64_t n_rows, bool decode);

}  // namespace sa
