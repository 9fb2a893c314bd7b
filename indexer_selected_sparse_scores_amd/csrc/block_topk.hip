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

// Steps 1 and 2 for one row: the key of every block's best score (from the row's scores, or from the
// maxima of its 64-token spans when pmax != nullptr) and the `kept` best blocks, written ascending to
// sh.kept.  Every thread of the workgroup calls it; it ends with a barrier.
template <int kW, class Sh>
__device__ __forceinline__ void select_kept_blocks(Sh &sh, const float *__restrict__ row, const uint32_t *__restrict__ pmax,
                                   int64_t n, int bs_shift, int kept, int n_blk)
{
    constexpr int kThreads = kW * kWave;
    const int tid = threadIdx.x;
    const int bs = 1 << bs_shift;
    for (int j = tid; j < kBins; j += kThreads) sh.hist[j] = 0;
    if (bs > kWave)
        for (int j = tid; j < n_blk; j += kThreads) sh.key[j] = 0;
    __syncthreads();

    // 1. block maxima
    if (pmax) {
        // from the maxima of the 64-token spans (block_size >= 64): block j covers spans
        // j * bs / 64 .. (j + 1) * bs / 64 - 1
        const int n64 = (int)((n + kWave - 1) / kWave), sh64 = bs_shift - 6;
        const uint32_t *prow = pmax;
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
        topk::select_and_emit_inline<kW>(sh.sel, BlockKeys{sh.key}, n_blk, sh.bin, sh.above, kept, sh.kept);
    }
    __syncthreads();
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

    select_kept_blocks<kWaves>(sh, row, pmax ? pmax + r * pmax_ld : nullptr, n, bs_shift, kept, n_blk);

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
        topk::select_and_emit_inline<kWaves>(sh.sel, cand, n_c, sh.bin, sh.above, m, dst);
    }
    for (int64_t i = m + tid; i < idx_ld; i += kThreads) dst[i] = -1;
}

// ---------------------------------------------------------------------------------------
// Two-tier prefill, second pass (bf16, H_I = 64, d_I = 128, blocks of a multiple of 64 tokens): the fused
// prefill kernel has left, for every row with more than n_blocks blocks, the order key of its best score
// in each 64-key tile.  One workgroup per row picks the kept blocks from those keys, scores only their
// tokens -- q of the row and its head weights in LDS, each wave taking 32 candidates at a time as the B
// operand of v_mfma_f32_32x32x16_bf16, with the fused kernel's k-step and epilogue order, so that every
// score equals the one the first pass saw bit for bit -- and selects the top k of them.
// ---------------------------------------------------------------------------------------
constexpr int kRH = 64;   // index heads
constexpr int kRD = 128;  // index head width
constexpr int kRWaves = 4;
constexpr int kRThreads = kRWaves * kWave;

struct RescoreShared {
    uint4 qf[2 * (kRD / 16) * kWave];     // q fragment (mt, ks) of lane l at (8 mt + ks) * 64 + l (16 KB)
    float wv[kRH];
    alignas(16) uint32_t hist[kBins];
    int32_t kept[kBlockSelectMaxKept];
    topk::SelectShared<kRWaves> sel;
    int bin, above;
};

// The selection helpers' view of the row's shared state; the key array (block keys, then candidate
// keys) is dynamic LDS sized to the call's largest need, so that several rows share a CU.
struct RescoreView {
    uint32_t *key;
    uint32_t *hist;
    int32_t *kept;
    topk::SelectShared<kRWaves> &sel;
    int &bin;
    int &above;
};

__global__ __launch_bounds__(kRThreads) void block_rescore_topk_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w, const uint16_t *__restrict__ k_idx,
    const int32_t *__restrict__ table, int64_t n_pages, int64_t L, int64_t pos0, int32_t topk, int32_t bs_shift,
    int32_t n_blocks, const uint32_t *__restrict__ bkeys, int64_t bkeys_ld, int32_t *__restrict__ idx)
{
    __shared__ RescoreShared sh;
    extern __shared__ __attribute__((aligned(16))) uint32_t key_lds[];
    RescoreView v{key_lds, sh.hist, sh.kept, sh.sel, sh.bin, sh.above};
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int64_t n = pos0 + r + 1;  // visible keys of the row
    int32_t *dst = idx + r * topk;
    const int bs = 1 << bs_shift;
    const int n_blk = (int)((n + bs - 1) >> bs_shift);
    const int kept = n_blocks < n_blk ? n_blocks : n_blk;
    if (kept < n_blk) {
        select_kept_blocks<kRWaves>(v, nullptr, bkeys + r * bkeys_ld, n, bs_shift, kept, n_blk);
    } else {
        for (int j = tid; j < n_blk; j += kRThreads) sh.kept[j] = j;
        __syncthreads();
    }
    const int last = sh.kept[kept - 1];
    const int n_c = (kept << bs_shift) - (last == n_blk - 1 ? (int)(((int64_t)n_blk << bs_shift) - n) : 0);
    const KeptTokens cand{key_lds, sh.kept, bs_shift};
    const int m = topk < n_c ? topk : n_c;
    if (m == n_c) {  // every candidate is selected: nothing to score
        for (int j = tid; j < n_c; j += kRThreads) dst[j] = cand.i(j);
        for (int j = n_c + tid; j < topk; j += kRThreads) dst[j] = -1;
        return;
    }

    // q fragments and head weights of the row
    {
        const uint16_t *qr = q_idx + r * (int64_t)kRH * kRD;
#pragma unroll
        for (int u = 0; u < 2 * (kRD / 16) * kWave / kRThreads; ++u) {
            const int f = tid + u * kRThreads, l = f % kWave, mk = f / kWave;
            sh.qf[f] = load16(qr + (32 * (mk / 8) + l % 32) * kRD + 16 * (mk % 8) + 8 * (l / 32));
        }
        if (tid < kRH) sh.wv[tid] = w[r * kRH + tid];
        for (int j = tid; j < kBins; j += kRThreads) sh.hist[j] = 0;
    }
    __syncthreads();
    // this lane's 32 head weights, in the order of its accumulator registers: register g of lane l is
    // head 32 mt + 8 (g / 4) + 4 (l / 32) + g % 4
    float wr[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int g = 0; g < 16; ++g) wr[mt][g] = sh.wv[32 * mt + 8 * (g / 4) + 4 * (lane / 32) + g % 4];

    // 32 candidates per wave at a time (bs >= 64: a group of 32 lies inside one block)
    const int n_groups = (n_c + 31) / 32;
#pragma unroll 1
    for (int grp = wave; grp < n_groups; grp += kRWaves) {
        const int j = 32 * grp + lane % 32;
        const bool ok = j < n_c;
        const int64_t tok = cand.i(ok ? j : 32 * grp);
        int64_t krow = tok;
        bool page_ok = true;
        if (table) {
            const int32_t pg = table[tok / 64];
            page_ok = pg >= 0 && pg < n_pages;
            krow = (int64_t)(page_ok ? pg : 0) * 64 + tok % 64;
        }
        const uint16_t *src = k_idx + krow * kRD + 8 * (lane / 32);
        bf16x8 b[kRD / 16];
#pragma unroll
        for (int ks = 0; ks < kRD / 16; ++ks) b[ks] = as_bf16x8(load16(src + 16 * ks));
        f32x16 acc0, acc1;
#pragma unroll
        for (int ks = 0; ks < kRD / 16; ++ks) {
            const bf16x8 a0 = as_bf16x8(sh.qf[ks * kWave + lane]);
            const bf16x8 a1 = as_bf16x8(sh.qf[(8 + ks) * kWave + lane]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[ks], ks == 0 ? f32x16{} : acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[ks], ks == 0 ? f32x16{} : acc1, 0, 0, 0);
        }
        float p = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            p = fmaf(wr[0][g], relu(acc0[g]), p);
            p = fmaf(wr[1][g], relu(acc1[g]), p);
        }
        // lanes l and l ^ 32 hold the two halves of the head sum of candidate j
        float score = p + __shfl_xor(p, 32);
        if (!page_ok) score = -__builtin_inff();
        if (lane < 32 && ok) {
            const uint32_t key = order_key(score);
            key_lds[j] = key;
            atomicAdd(&sh.hist[key >> kBinShift], 1u);
        }
    }
    __syncthreads();
    if (tid < kWave) {
        int above;
        const int bin = topk::threshold_bin(sh.hist, m, &above, nullptr);
        if (tid == 0) {
            sh.bin = bin;
            sh.above = above;
        }
    }
    __syncthreads();
    topk::select_and_emit_inline<kRWaves>(sh.sel, cand, n_c, sh.bin, sh.above, m, dst);
    for (int j = m + tid; j < topk; j += kRThreads) dst[j] = -1;
}

}  // namespace

hipError_t launch_block_rescore_topk(sa_handle_s &h, const void *q_idx, const float *w, const void *k_idx,
                                     const int32_t *table, int64_t n_pages, int64_t L, int64_t pos0, int32_t topk,
                                     int32_t block_size, int32_t n_blocks, const uint32_t *bkeys, int64_t bkeys_ld,
                                     int32_t *idx, hipStream_t st)
{
    if (L <= 0) return hipSuccess;
    int shift = 0;
    while ((1 << shift) < block_size) ++shift;
    // the key array holds a row's block keys, then its candidates' keys
    const int64_t n_blk_max = (pos0 + L + block_size - 1) / block_size;
    const int64_t items = n_blk_max > (int64_t)n_blocks * block_size ? n_blk_max : (int64_t)n_blocks * block_size;
    const size_t dyn = (size_t)items * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(block_rescore_topk_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    KernelTimer timer(h, SA_KERNEL_TOPK, st);
    hipLaunchKernelGGL(block_rescore_topk_kernel, dim3((unsigned)L), dim3(kRThreads), dyn, st,
                       reinterpret_cast<const uint16_t *>(q_idx), w, reinterpret_cast<const uint16_t *>(k_idx), table,
                       n_pages, L, pos0, topk, shift, n_blocks, bkeys, bkeys_ld, idx);
    return hipGetLastError();
}

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
