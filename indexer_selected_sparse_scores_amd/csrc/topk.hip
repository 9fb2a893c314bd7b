// Per-row top-k selection on gfx950.
//
// For each row: the min(k, n) columns with the largest scores among the first n, ties
// going to the lower column -- the per-query token selection of "Sparse Attention and RL
// Optimization: Three Technical Breakthroughs in LLM Post-Training", section 2.3 (and the
// `topk` step of its section 2.5 pseudocode).
//
// One 256-thread workgroup per row.  Scores are mapped to order-preserving uint32 keys and
// the k-th largest key is found exactly by a most-significant-digit radix select: four
// passes of 8-bit digits, each a 256-bin histogram in LDS of the keys that still match
// the digits fixed so far, followed by a workgroup scan that picks the digit holding the
// k-th element.  A final ordered pass emits every key above the threshold plus the first
// `need` keys equal to it (the lowest columns), so the output is exact, deterministic and
// ascending.  No score is written back; the row is only read.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;  // consecutive elements per thread in the ordered pass

// Inclusive prefix sum over the 256 threads of the workgroup; returns the inclusive sum
// for this thread and the workgroup total in *total.  Uses 4 ints of LDS.
__device__ __forceinline__ int block_inclusive_scan(int v, int *wave_sums, int *total)
{
    const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == kWave - 1) wave_sums[wave] = v;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) {
        int ws = wave_sums[i];
        if (i < wave) before += ws;
        all += ws;
    }
    __syncthreads();  // wave_sums may be reused right after
    *total = all;
    return v + before;
}

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(
    const float *__restrict__ scores, int64_t ld, int64_t cols, const int32_t *__restrict__ valid_len,
    int64_t causal_row0, const int32_t *__restrict__ k_per_row, int32_t k, int32_t *__restrict__ idx,
    int64_t idx_ld, uint32_t *err)
{
    __shared__ uint32_t hist[256];
    __shared__ int wave_sums[kThreads / kWave];
    __shared__ uint32_t sh_digit;
    __shared__ int sh_need;

    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    int32_t *dst = idx + row * idx_ld;

    int64_t n;
    if (valid_len) {
        n = valid_len[row];
    } else {
        n = causal_row0 + row + 1;
        if (n > cols) n = cols;
    }
    const int64_t kr = k_per_row ? (int64_t)k_per_row[row] : (int64_t)k;
    if (n < 1 || n > cols || kr < 1 || kr > k) {
        if (tid == 0) flag_error(err, SA_DEVERR_TOPK);
        for (int64_t i = tid; i < idx_ld; i += kThreads) dst[i] = -1;
        return;
    }
    const int64_t m = kr < n ? kr : n;
    if (m == n) {  // every visible column is selected
        for (int64_t i = tid; i < idx_ld; i += kThreads) dst[i] = i < n ? (int32_t)i : -1;
        return;
    }
    const float *src = scores + row * ld;

    // ---- radix select of the m-th largest key ------------------------------------------
    uint32_t prefix = 0, mask = 0;
    int need = (int)m;  // how many of the keys matching `prefix` still have to be taken
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int64_t s = tid; s < n; s += kThreads) {
            uint32_t key = order_key(src[s]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFFu], 1u);
        }
        __syncthreads();
        // thread t looks at digit 255 - t, so the prefix over threads counts the keys
        // whose digit is >= that digit
        const uint32_t d = 255u - (uint32_t)tid;
        const int c = (int)hist[d];
        int total;
        const int incl = block_inclusive_scan(c, wave_sums, &total);
        const int excl = incl - c;
        if (excl < need && need <= incl) {
            sh_digit = d;
            sh_need = need - excl;
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 0xFFu << shift;
        need = sh_need;
        __syncthreads();
    }
    const uint32_t tau = prefix;  // exact key of the m-th largest element

    // ---- ordered emit: keys > tau, then the first `need` keys == tau --------------------
    int out_before = 0, eq_before = 0;
    const int64_t tile = (int64_t)kThreads * kPerThread;
#pragma unroll 1
    for (int64_t base = 0; base < n; base += tile) {
        const int64_t s0 = base + (int64_t)tid * kPerThread;
        uint32_t keys[kPerThread];
        int n_eq = 0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            int64_t s = s0 + i;
            keys[i] = s < n ? order_key(src[s]) : 0u;
            n_eq += (s < n && keys[i] == tau) ? 1 : 0;
        }
        int eq_total;
        int eq_rank = block_inclusive_scan(n_eq, wave_sums, &eq_total) - n_eq + eq_before;
        bool take[kPerThread];
        int n_take = 0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            int64_t s = s0 + i;
            bool valid = s < n;
            bool gt = valid && keys[i] > tau;
            bool eq = valid && keys[i] == tau;
            take[i] = gt || (eq && eq_rank < need);
            eq_rank += eq ? 1 : 0;
            n_take += take[i] ? 1 : 0;
        }
        int take_total;
        int pos = block_inclusive_scan(n_take, wave_sums, &take_total) - n_take + out_before;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
            if (take[i] && pos < m) dst[pos++] = (int32_t)(s0 + i);
        out_before += take_total;
        eq_before += eq_total;
    }
    for (int64_t i = m + tid; i < idx_ld; i += kThreads) dst[i] = -1;
}

}  // namespace

hipError_t launch_topk(sa_handle_s &h, const float *scores, int64_t ld, int64_t rows, int64_t cols,
                       const int32_t *valid_len, int64_t causal_row0, const int32_t *k_per_row,
                       int32_t k, int32_t *idx, int64_t idx_ld, uint32_t *err, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    KernelTimer timer(h, SA_KERNEL_TOPK, st);
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, scores, ld,
                       cols, valid_len, causal_row0, k_per_row, k, idx, idx_ld, err);
    return hipGetLastError();
}

}  // namespace sa
