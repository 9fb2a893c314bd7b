// Query rows against paged caches: chunked prefill, varlen batches and multi-token decode.
//
// "Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and Verifiable
// Synthetic Data", section 2.3: the selection composes with paged KV management, and a query
// reads only its selected entries; "Sparse Attention and RL Optimization: Three Technical
// Breakthroughs in LLM Post-Training", section 2.5: a query at position p looks back at the
// tokens s <= p of its own sequence.  Each query row names its sequence and position; this
// kernel checks both once and writes the per-row arrays the indexer, top-k and attention kernels
// read (block-table row, visible length p + 1, budget), so that no later kernel can index the
// block table with an unchecked row.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

namespace {

__global__ void paged_rows_kernel(const int32_t *__restrict__ row_seq, const int32_t *__restrict__ row_pos,
                                  int64_t T, int32_t n_seqs, int32_t max_ctx, int32_t topk, int32_t *__restrict__ seq,
                                  int32_t *__restrict__ ctx, int32_t *__restrict__ budget, uint32_t *err)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const int32_t b = row_seq[t], p = row_pos[t];
    const bool ok = b >= 0 && b < n_seqs && p >= 0 && p < max_ctx;
    if (!ok) flag_error(err, SA_DEVERR_ROW);
    seq[t] = ok ? b : 0;
    ctx[t] = ok ? p + 1 : 0;  // 0: every later kernel skips the row
    budget[t] = topk;
}

}  // namespace

hipError_t launch_paged_rows(sa_handle_s &h, const int32_t *row_seq, const int32_t *row_pos, int64_t T,
                             int32_t n_seqs, int32_t max_ctx, int32_t topk, int32_t *seq, int32_t *ctx,
                             int32_t *budget, hipStream_t st)
{
    hipLaunchKernelGGL(paged_rows_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, row_seq, row_pos, T,
                       n_seqs, max_ctx, topk, seq, ctx, budget, h.d_err);
    return hipGetLastError();
}

}  // namespace sa
