/*
 * Reference oracle for indexer-selected sparse attention -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct CPU definition of what the GPU
 * library computes.  Only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it.  It shares no code, header, table or helper with the
 * HIP library; it never calls into it, and the library never calls into this.
 *
 * Everything is accumulated in double.  Inputs are float32 arrays (bf16 inputs are
 * widened to float32 exactly by the caller, then to double here).  No blocking, no
 * fusion, no reordering beyond the definitions cited at each function.
 *
 * Sources (the pages the method is defined on):
 *   [P1] "Sparse Attention and RL Optimization: Three Technical Breakthroughs in LLM
 *        Post-Training" -- section 2.2 (indexer score formula and its design points),
 *        section 2.3 (per-query top-k token selection), section 2.5 (pseudocode of the
 *        indexer -> causal mask -> top-k -> gather -> softmax attention pipeline).
 *   [P2] "A Guide to Sparse Attention and Efficient Reinforcement Learning in LLM
 *        Long-Context Inference" -- section 1 (the model keeps multi-head latent
 *        attention), section 1.1 (two-tier block -> token selection).
 *   [P3] "Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning,
 *        and Verifiable Synthetic Data" -- section 2.2 (two-stage design), section 2.3
 *        (decode reads only the selected k KV entries; composes with paged KV
 *        management), section 2.4 (reference pseudocode: attention logits scaled by
 *        1/sqrt(d)).
 *
 * Readings where the pages are silent:
 *   - causal visibility is s <= t: the query sees itself, so row 0 is never empty;
 *   - one index key k(s) per token, shared by all index heads ([P1] 2.2 gives k(s) no
 *     head index, and the 2.5 pseudocode has a single i_k per token);
 *   - no scale and no normalisation inside the indexer; w may be negative;
 *   - ties in top-k are broken toward the lower token index;
 *   - fewer than k visible tokens: select all visible ones and pad with -1 (taking
 *     top-k over masked -inf entries, as the pseudocode would, attends to the future);
 *   - the attention scale is 1/sqrt(d_qk), the key width; the caller passes it in.
 *
 * Parity status: every function below is pinned by the CPU tests (hand-worked golden
 * values, library special cases, closed forms, brute-force ranking).  None is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------
 * Indexer score, [P1] section 2.2:
 *     I(t,s) = sum_j w(t,j) * ReLU( q(t,j) . k(s) )
 * For query row i (one query token with H_I index heads of width d_I) and every key
 * s in [0, n_k): if s < visible[i] the score above, otherwise -infinity (the causal
 * mask of the [P1] section 2.5 pseudocode: only look-back is allowed).
 * abs_out (optional) receives A(t,s) = sum_j |w(t,j)| * ReLU(q(t,j) . k(s)), the sum of
 * the absolute values of the terms, used to scale floating-point tolerances.
 * ---------------------------------------------------------------------------------- */
void orc_indexer_scores(const float *q,         /* [n_q, H_I, d_I] */
                        const float *w,         /* [n_q, H_I]      */
                        const float *k,         /* [n_k, d_I]      */
                        const int64_t *visible, /* [n_q]           */
                        int64_t n_q, int64_t n_k, int H_I, int d_I,
                        double *out,            /* [n_q, n_k]      */
                        double *abs_out)        /* [n_q, n_k] or NULL */
{
    /* one (query, key) pair per iteration, so a single decode query still spreads
       over every thread */
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t pair = 0; pair < n_q * n_k; ++pair) {
        int64_t i = pair / n_k, s = pair % n_k;
        double score = -INFINITY, abs_score = -INFINITY;
        if (s < visible[i]) {
            score = 0.0;
            abs_score = 0.0;
            for (int j = 0; j < H_I; ++j) {
                double dot = 0.0;
                for (int c = 0; c < d_I; ++c)
                    dot += (double)q[(i * H_I + j) * (int64_t)d_I + c] *
                           (double)k[s * (int64_t)d_I + c];
                double relu = dot > 0.0 ? dot : 0.0;
                double wj = (double)w[i * H_I + j];
                score += wj * relu;
                abs_score += fabs(wj) * relu;
            }
        }
        out[pair] = score;
        if (abs_out) abs_out[pair] = abs_score;
    }
}

/* ------------------------------------------------------------------------------------
 * Per-query top-k, [P1] section 2.3 and the `topk` step of the section 2.5 pseudocode:
 * among the visible keys s < visible[i], order by (score descending, index ascending)
 * and keep the first m = min(k_i, visible[i]); the remaining k_max - m slots are -1.
 * The output row lists the selected indices in that rank order.
 * ---------------------------------------------------------------------------------- */
typedef struct {
    double score;
    int64_t index;
} orc_cand;

static int orc_cand_rank_order(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *b = (const orc_cand *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->index < b->index) ? -1 : (a->index > b->index);
}

void orc_topk(const double *scores,     /* [n_q, ld]                        */
              int64_t ld,
              const int64_t *visible,   /* [n_q]                            */
              const int32_t *k_per_row, /* [n_q] or NULL (then k_max each)  */
              int64_t n_q, int32_t k_max,
              int32_t *idx)             /* [n_q, k_max]                     */
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_q; ++i) {
        int64_t n = visible[i];
        int64_t k = k_per_row ? k_per_row[i] : k_max;
        int64_t m = k < n ? k : n;
        orc_cand *c = (orc_cand *)malloc((size_t)(n > 0 ? n : 1) * sizeof(orc_cand));
        for (int64_t s = 0; s < n; ++s) {
            c[s].score = scores[i * ld + s];
            c[s].index = s;
        }
        qsort(c, (size_t)n, sizeof(orc_cand), orc_cand_rank_order);
        for (int64_t r = 0; r < k_max; ++r)
            idx[i * k_max + r] = r < m ? (int32_t)c[r].index : -1;
        free(c);
    }
}

/* ------------------------------------------------------------------------------------
 * Two-tier (block -> token) selection, [P2] "A Guide to Sparse Attention and Efficient
 * Reinforcement Learning in LLM Long-Context Inference", section 1.1 (fine-grained token
 * selection): the history is cut into fixed-size blocks, a few high-value blocks are kept
 * on the strength of the indexer scores, and token-level selection then runs inside the
 * kept blocks only.  Readings (the page fixes none of these details):
 *   - block j holds the tokens s with s / block_size == j (aligned to position 0), and
 *     only its visible tokens s < visible[i] belong to it, so the last block may be short;
 *   - a block's score is the largest indexer score among its visible tokens;
 *   - blocks are ranked by (block score descending, block index ascending) and the first
 *     min(n_blocks, number of visible blocks) are kept;
 *   - the candidates are the visible tokens of the kept blocks; they are ranked by
 *     (score descending, token index ascending) and the first min(k_i, candidates) are
 *     selected; the remaining k_max slots are -1.
 * The output row lists the selected indices in rank order.  blocks_out (optional,
 * [n_q, n_blocks]) receives the kept block indices in rank order, -1 padded.
 * ---------------------------------------------------------------------------------- */
void orc_block_topk(const double *scores,     /* [n_q, ld]                       */
                    int64_t ld,
                    const int64_t *visible,   /* [n_q]                           */
                    const int32_t *k_per_row, /* [n_q] or NULL (then k_max each) */
                    int64_t n_q, int32_t k_max,
                    int64_t block_size, int64_t n_blocks,
                    int32_t *idx,             /* [n_q, k_max]                    */
                    int32_t *blocks_out)      /* [n_q, n_blocks] or NULL         */
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_q; ++i) {
        int64_t n = visible[i];
        int64_t k = k_per_row ? k_per_row[i] : k_max;
        int64_t n_blk = (n + block_size - 1) / block_size;
        int64_t kept = n_blocks < n_blk ? n_blocks : n_blk;
        orc_cand *blk = (orc_cand *)malloc((size_t)(n_blk > 0 ? n_blk : 1) * sizeof(orc_cand));
        char *chosen = (char *)calloc((size_t)(n_blk > 0 ? n_blk : 1), 1);
        orc_cand *c = (orc_cand *)malloc((size_t)(n > 0 ? n : 1) * sizeof(orc_cand));
        for (int64_t j = 0; j < n_blk; ++j) {
            double best = -INFINITY;
            for (int64_t s = j * block_size; s < (j + 1) * block_size && s < n; ++s)
                if (scores[i * ld + s] > best) best = scores[i * ld + s];
            blk[j].score = best;
            blk[j].index = j;
        }
        qsort(blk, (size_t)n_blk, sizeof(orc_cand), orc_cand_rank_order);
        for (int64_t r = 0; r < kept; ++r) chosen[blk[r].index] = 1;
        if (blocks_out)
            for (int64_t r = 0; r < n_blocks; ++r)
                blocks_out[i * n_blocks + r] = r < kept ? (int32_t)blk[r].index : -1;
        int64_t n_c = 0;
        for (int64_t s = 0; s < n; ++s) {
            if (!chosen[s / block_size]) continue;
            c[n_c].score = scores[i * ld + s];
            c[n_c].index = s;
            ++n_c;
        }
        qsort(c, (size_t)n_c, sizeof(orc_cand), orc_cand_rank_order);
        int64_t m = k < n_c ? k : n_c;
        for (int64_t r = 0; r < k_max; ++r)
            idx[i * k_max + r] = r < m ? (int32_t)c[r].index : -1;
        free(blk);
        free(chosen);
        free(c);
    }
}

/* ------------------------------------------------------------------------------------
 * Softmax attention over a selected set of rows, [P1] section 2.5 (`gather` then
 * softmax(q k_sel^T / sqrt(d)) v_sel) and [P3] section 2.4 (the same with an explicit
 * logits step).  For query row i and head h, with kv head g = h * H_kv / H:
 *     l_s   = scale * sum_c q[i,h,c] * K[s,g,c]          for s in sel(i)
 *     mu    = max_s l_s
 *     O     = sum_s exp(l_s - mu) V[s,g,:] / sum_s exp(l_s - mu)
 *     LSE   = mu + log sum_s exp(l_s - mu)
 * sel(i) is the set of non-negative entries of idx row i.  If V is NULL the value row
 * is the first d_v columns of the key row (one shared latent row per token, the MLA
 * layout that [P2] "A Guide to Sparse Attention and Efficient Reinforcement Learning
 * in LLM Long-Context Inference", section 1, says the model keeps).
 * A row with an empty selection gets O = 0 and LSE = -infinity.
 * ---------------------------------------------------------------------------------- */
void orc_attention(const float *q,      /* [n_q, H, d_qk]          */
                   const float *K,      /* [n_k, H_kv, d_qk]       */
                   const float *V,      /* [n_k, H_kv, d_v] or NULL */
                   const int32_t *idx,  /* [n_q, idx_ld]           */
                   int64_t idx_ld, int64_t n_q, int64_t n_k,
                   int H, int H_kv, int d_qk, int d_v, double scale,
                   double *out,         /* [n_q, H, d_v]           */
                   double *lse)         /* [n_q, H] or NULL        */
{
    (void)n_k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_q; ++i) {
        const int32_t *sel = idx + i * idx_ld;
        double *logit = (double *)malloc((size_t)(idx_ld > 0 ? idx_ld : 1) * sizeof(double));
        for (int h = 0; h < H; ++h) {
            int g = (int)((int64_t)h * H_kv / H);
            const float *qh = q + (i * H + h) * (int64_t)d_qk;
            double mu = -INFINITY;
            int64_t count = 0;
            for (int64_t r = 0; r < idx_ld; ++r) {
                if (sel[r] < 0) continue;
                const float *kr = K + ((int64_t)sel[r] * H_kv + g) * d_qk;
                double dot = 0.0;
                for (int c = 0; c < d_qk; ++c) dot += (double)qh[c] * (double)kr[c];
                logit[r] = scale * dot;
                if (logit[r] > mu) mu = logit[r];
                ++count;
            }
            double *o = out + (i * H + h) * (int64_t)d_v;
            for (int c = 0; c < d_v; ++c) o[c] = 0.0;
            if (count == 0) {
                if (lse) lse[i * H + h] = -INFINITY;
                continue;
            }
            double denom = 0.0;
            for (int64_t r = 0; r < idx_ld; ++r) {
                if (sel[r] < 0) continue;
                double p = exp(logit[r] - mu);
                denom += p;
                const float *vr = V ? V + ((int64_t)sel[r] * H_kv + g) * d_v
                                    : K + ((int64_t)sel[r] * H_kv + g) * d_qk;
                for (int c = 0; c < d_v; ++c) o[c] += p * (double)vr[c];
            }
            for (int c = 0; c < d_v; ++c) o[c] /= denom;
            if (lse) lse[i * H + h] = mu + log(denom);
        }
        free(logit);
    }
}

/* ------------------------------------------------------------------------------------
 * Threads the OpenMP runtime will use (reported next to timings of this oracle).
 * ---------------------------------------------------------------------------------- */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads later OpenMP loops of this oracle use (n >= 1; timing aid, no effect on results). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
