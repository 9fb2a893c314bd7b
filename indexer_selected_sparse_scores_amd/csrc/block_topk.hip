// Two-tier (block -> token) selection on gfx950.
//
// "A Guide to Sparse Attention and Efficient Reinforcement Learning in LLM Long-Context
// Inference", section 1.1 (fine-grained token selection): the history is cut into fixed-size
// blocks, a few high-value blocks are kept on the strength of the indexer scores, and the
// token-level selection then runs inside the kept blocks only.  Readings: block j is the visible
// tokens s with s / block_size == j; its score is the largest score among them; blocks and
// tokens both rank by (score desc, index asc), the tie rule of "Sparse Attention and RL
// Optimization: Three Technical Breakthroughs in LLM Post-Training", section 2.3.
//
// One 1024-thread workgroup per row, everything in LDS (about 80 KB):
//  1. block maxima: coalesced loads of the row's scores as order-preserving keys, a max over
//     each block's lanes (blocks of up to 64 tokens live inside one wave; longer ones are
//     combined with LDS atomics) -- or, when the producer of the scores also wrote the maxima of
//     each 64-token span (the paged decode indexer does, one per page), a combination of those --
//     and a 2048-bin histogram of the block keys;
//  2. the kept blocks: the threshold bin of the n_blocks-th block key, an MSD radix select and
//     an ordered emit of the kept block ids in ascending order (the shared top-k helpers);
//  3. the candidates: the visible tokens of the kept blocks, in ascending token order (only the
//     last visible block can be short, and it is the highest block), keys and a histogram in
//     LDS; the same select then writes the selected tokens in ascending order.
#include "sa_device.hpp"
#include "sa_internal.hpp"
#include "topk_device.hpp"

namespace sa {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * kWave;
using topk::kBinShift;
using topk::kBins;

struct BlockTopkShared {
    uint32_t key[kBlockSelectMaxItems];  // block keys, then candidate token keys
    alignas(16) uint32_t hist[kBins];    // read 16 bytes at a time by threshold_bin
    int32_t kept[kBlockSelectMaxKept];   // kept block ids, ascending
    topk::SelectShared<kWaves> sel;
    int bin, above;
};

// Block j of the row is element j (its key is the block's best score key).
struct BlockKeys {
    const uint32_t *key;
    __device__ uint32_t k(int j) const { return key[j]; }
    __device__ int32_t i(int j) const { return j; }
};

// Candidate j is token (kept[j / bs]) * bs + j % bs.
struct KeptTokens {
    const uint32_t *key;
    const int32_t *kept;
    int shift;
    __device__ uint32_t k(int j) const { return key[j]; }
    __device__ int32_t i(int j) const
    {
        return (kept[j >> shift] << shift) | (j & ((1 << shift) - 1));
    }
};

// The wave's largest key over each aligned group of `g` lanes (g a power of two <= 64).
__device__ __forceinline__ uint32_t group_max(uint32_t x, int g)
{
    for (int off = 1; off < g; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)x, off);
        x = x > y ? x : y;
    }
    return x;
}

__global__ __launch_bounds__(kThreads) void block_topk_rows_kernel(
    const float *__restrict__ scores, int64_t ld, int64_t cols, const int32_t *__restrict__ valid_len,
    int64_t causal_row0, const int32_t *__restrict__ k_per_row, int32_t k, int32_t bs_shift,
    int32_t n_blocks, const uint32_t *__restrict__ pmax, int64_t pmax_ld, int32_t *__restrict__ idx,
    int64_t idx_ld, uint32_t *err)
{
    __shared__ BlockTopkShared sh;
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const float *row = scores + r * ld;
    int32_t *dst = idx + r * idx_ld;

    int64_t n;
    if (valid_len) {
        n = valid_len[r];
    } else {
        n = causal_row0 + r + 1;
        if (n > cols) n = cols;
    }
    const int64_t kr = k_per_row ? (int64_t)k_per_row[r] : (int64_t)k;
    if (n < 1 || n > cols || kr < 1 || kr > k) {
        if (tid == 0) flag_error(err, SA_DEVERR_TOPK);
        for (int64_t i = tid; i < idx_ld; i += kThreads) dst[i] = -1;
        return;
    }
    const int bs = 1 << bs_shift;
    const int n_blk = (int)((n + bs - 1) >> bs_shift);  // <= kBlockSelectMaxItems (host check)
    const int kept = n_blocks < n_blk ? n_blocks : n_blk;

    for (int j = tid; j < kBins; j += kThreads) sh.hist[j] = 0;
    if (bs > kWave)
        for (int j = tid; j < n_blk; j += kThreads) sh.key[j] = 0;
    __syncthreads();

    // 1. block maxima
    if (pmax) {
        // from the maxima of the 64-token spans (block_size >= 64): block j covers spans
        // j * bs / 64 .. (j + 1) * bs / 64 - 1
        const int n64 = (int)((n + kWave - 1) / kWave), sh64 = bs_shift - 6;
        const uint32_t *prow = pmax + r * pmax_ld;
        for (int j = tid; j < n64; j += kThreads) {
            const uint32_t x = prow[j];
            if (sh64 == 0) sh.key[j] = x;
            else atomicMax(&sh.key[j >> sh64], x);
        }
    } else {
        // from the scores, four rounds of loads in flight.  A block of <= 64 tokens is a group of
        // lanes of one wave, led by the lane holding its first token (s % bs == 0, since each round
        // starts at a multiple of 1024); longer blocks combine their waves' maxima with atomics.
        const int g = bs < kWave ? bs : kWave;
        for (int64_t base = 0; base < n; base += 4 * kThreads) {
            uint32_t x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t s = base + u * kThreads + tid;
                x[u] = s < n ? order_key(row[s]) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t s = base + u * kThreads + tid;
                const uint32_t m = group_max(x[u], g);
                if ((tid & (g - 1)) == 0 && s < n) {
                    if (bs <= kWave) sh.key[s >> bs_shift] = m;
                    else atomicMax(&sh.key[s >> bs_shift], m);
                }
            }
        }
    }
    __syncthreads();
    for (int j = tid; j < n_blk; j += kThreads) atomicAdd(&sh.hist[sh.key[j] >> kBinShift], 1u);
    __syncthreads();

    // 2. the kept blocks, ascending
    if (kept == n_blk) {
        for (int j = tid; j < n_blk; j += kThreads) sh.kept[j] = j;
    } else {
        if (tid < kWave) {
            int above;
            const int bin = topk::threshold_bin(sh.hist, kept, &above, nullptr);
            if (tid == 0) {
                sh.bin = bin;
                sh.above = above;
            }
        }
        __syncthreads();
        topk::select_and_emit<kWaves>(sh.sel, BlockKeys{sh.key}, n_blk, sh.bin, sh.above, kept, sh.kept);
    }
    __syncthreads();

    // 3. candidates: the visible tokens of the kept blocks, ascending
    const int last = sh.kept[kept - 1];
    const int n_c = (kept << bs_shift) - (last == n_blk - 1 ? (int)(((int64_t)n_blk << bs_shift) - n) : 0);
    for (int j = tid; j < kBins; j += kThreads) sh.hist[j] = 0;
    __syncthreads();
    const KeptTokens cand{sh.key, sh.kept, bs_shift};
    for (int j = tid; j < n_c; j += kThreads) {
        const uint32_t key = order_key(row[cand.i(j)]);
        sh.key[j] = key;
        atomicAdd(&sh.hist[key >> kBinShift], 1u);
    }
    __syncthreads();
    const int m = kr < n_c ? (int)kr : n_c;
    if (m == n_c) {
        for (int j = tid; j < n_c; j += kThreads) dst[j] = cand.i(j);
    } else {
        if (tid < kWave) {
            int above;
            const int bin = topk::threshold_bin(sh.hist, m, &above, nullptr);
            if (tid == 0) {
                sh.bin = bin;
                sh.above = above;
            }
        }
        __syncthreads();
        topk::select_and_emit<kWaves>(sh.sel, cand, n_c, sh.bin, sh.above, m, dst);
    }
    for (int64_t i = m + tid; i < idx_ld; i += kThreads) dst[i] = -1;
}

}  // namespace

hipError_t launch_block_topk(sa_handle_s &h, const float *scores, int64_t ld, int64_t rows, int64_t cols,
                             const int32_t *valid_len, int64_t causal_row0, const int32_t *k_per_row, int32_t k,
                             int32_t block_size, int32_t n_blocks, const uint32_t *pmax, int64_t pmax_ld,
                             int32_t *idx, int64_t idx_ld, uint32_t *err, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    int shift = 0;
    while ((1 << shift) < block_size) ++shift;
    if (block_size < kWave) pmax = nullptr;
    KernelTimer timer(h, SA_KERNEL_TOPK, st);
    hipLaunchKernelGGL(block_topk_rows_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, scores, ld, cols,
                       valid_len, causal_row0, k_per_row, k, shift, n_blocks, pmax, pmax_ld, idx, idx_ld, err);
    return hipGetLastError();
}

}  // namespace sa
