// Device building blocks of the exact per-row top-k shared by the prefill and decode kernels.
//
// Selection order: larger score first, ties to the lower token index -- the per-query
// token selection of "Sparse Attention and RL Optimization: Three Technical Breakthroughs in
// LLM Post-Training", section 2.3.  Scores are compared through order_key(), an order-
// preserving map of fp32 to uint32.  The top 11 key bits (2048 bins) give a histogram from
// which the bin holding the m-th largest score is found; the final choice inside that bin is
// an MSD radix select over the remaining 21 bits, and an ordered compaction emits the
// selection in ascending token order.
#pragma once

#include "sa_device.hpp"

namespace sa {
namespace topk {

constexpr int kBins = 2048;         // histogram bins over the key's top 11 bits
constexpr int kBinShift = 21;
constexpr int kCap = 8192;          // candidates held in LDS for the final selection
constexpr int kPerThread = 16;      // consecutive candidates per thread in ordered passes

// Workgroup-shared scratch of the selection helpers (kWaves waves).
template <int kWaves>
struct SelectShared {
    uint32_t radix[128];
    int wave_sums[kWaves];
    uint32_t digit;
    int need;
};

// Inclusive prefix sum over the 64 lanes of a wave (lane 0 first) on DPP: row shifts by 1, 2, 4
// and 8 within each 16-lane row (lanes shifted in from outside the row read 0), then the last
// lane of row 0 added into row 1 (and of row 2 into row 3), then lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Exclusive prefix sum over the kWaves * 64 threads (thread order); *total gets the sum.
template <int kWaves>
__device__ __forceinline__ int block_scan(int v, int *wave_sums, int *total)
{
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int x = wave_incl_scan(v);
    if (lane == kWave - 1) wave_sums[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int s = wave_sums[i];
        before += i < wave ? s : 0;
        all += s;
    }
    __syncthreads();
    *total = all;
    return x - v + before;
}

// One wave: the highest bin b of a 2048-bin histogram (LDS or global memory) such that the
// bins >= b hold at least m >= 1 entries.  Returns -1 if the whole histogram holds fewer than m.
// *above = entries in bins > b, *upto = entries in bins >= b (either may be NULL).  Every
// lane returns the same values.
__device__ __forceinline__ int threshold_bin(const uint32_t *hist, int m, int *above, int *upto)
{
    const int lane = lane_id();
    // lane l sums bins [kBins - 32 (l + 1), kBins - 32 l): lane 0 holds the top bins
    const uint32_t *hb = hist + kBins - 32 * (lane + 1);
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(hb + i);
        sum += (int)(v.x + v.y + v.z + v.w);
    }
    const int incl = wave_incl_scan(sum);
    const uint64_t hit = __ballot(incl >= m);
    if (hit == 0) {
        if (above) *above = 0;
        if (upto) *upto = __builtin_amdgcn_readlane(incl, kWave - 1);
        return -1;
    }
    // lane src's range holds the answer; its 32 bins, top first, go one per lane to lanes 0..31
    const int src = __builtin_ctzll(hit);
    const int base = __builtin_amdgcn_readlane(incl - sum, src);  // entries above that range
    const int top = kBins - 32 * src - 1;
    const int c = lane < 32 ? (int)hist[top - (lane & 31)] : 0;
    const int cum = base + wave_incl_scan(c);
    const int j = __builtin_ctzll(__ballot(lane < 32 && cum >= m));
    const int up = __builtin_amdgcn_readlane(cum, j);
    if (above) *above = up - __builtin_amdgcn_readlane(c, j);
    if (upto) *upto = up;
    return top - j;
}

// Candidate sources for select_and_emit: element j has key k(j) and token index i(j); the
// elements are in ascending token order.
struct LdsCands {
    const uint32_t *key;
    const int32_t *idx;
    __device__ uint32_t k(int j) const { return key[j]; }
    __device__ int32_t i(int j) const { return idx[j]; }
};
struct GlobalCands {
    const uint2 *c;  // (key, index)
    __device__ uint32_t k(int j) const { return c[j].x; }
    __device__ int32_t i(int j) const { return (int32_t)c[j].y; }
};
struct GlobalScores {
    const float *s;  // a score row; element j is token j
    __device__ uint32_t k(int j) const { return order_key(s[j]); }
    __device__ int32_t i(int j) const { return j; }
};

// Exact selection of the `need` largest keys among the n candidates whose top bits equal
// `bin` (the ones in higher bins are all taken: `above` of them), then an ordered emit of the
// m = above + need selected indices (ascending) into dst[0, m).  Candidates in lower bins are
// skipped.  Every thread of the workgroup calls this.  select_and_emit_inline is the body, for
// kernels with registers to spare (no call frame in scratch memory); select_and_emit keeps it out
// of line for kernels that hold many live registers around the call.
template <int kWaves, class Src>
__device__ __forceinline__ void select_and_emit_inline(SelectShared<kWaves> &sh, const Src &src, int n, int bin,
                                                       int above, int m, int32_t *dst)
{
    constexpr int kThreads = kWaves * kWave;
    const int tid = threadIdx.x;
    int need = m - above;  // >= 1
    uint32_t prefix = (uint32_t)bin << kBinShift, mask = 0xFFFFFFFFu << kBinShift;
#pragma unroll 1
    for (int shift = 14; shift >= 0; shift -= 7) {
        if (tid < 128) sh.radix[tid] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kThreads) {
            const uint32_t key = src.k(j);
            if ((key & mask) == prefix) atomicAdd(&sh.radix[(key >> shift) & 127u], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l looks at digits 127 - 2l and 126 - 2l (descending)
            const int c_hi = (int)sh.radix[127 - 2 * tid], c_lo = (int)sh.radix[126 - 2 * tid];
            const int c = c_hi + c_lo;
            const int incl = wave_incl_scan(c);
            const int excl = incl - c;
            if (excl < need && need <= incl) {
                if (need <= excl + c_hi) {
                    sh.digit = 127u - 2u * tid;
                    sh.need = need - excl;
                } else {
                    sh.digit = 126u - 2u * tid;
                    sh.need = need - excl - c_hi;
                }
            }
        }
        __syncthreads();
        prefix |= sh.digit << shift;
        mask |= 127u << shift;
        need = sh.need;
        __syncthreads();
    }
    const uint32_t tau = prefix;  // exact key of the m-th largest score

    // ordered emit: every key > tau, then the first `need` keys == tau (lowest indices)
    int eq_before = 0, out_before = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += kThreads * kPerThread) {
        const int j0 = base + tid * kPerThread;
        uint32_t gt = 0, eq = 0;  // bit i: candidate j0 + i
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int j = j0 + i;
            if (j < n) {
                const uint32_t key = src.k(j);
                gt |= (key > tau ? 1u : 0u) << i;
                eq |= (key == tau ? 1u : 0u) << i;
            }
        }
        int eq_total;
        int eq_rank = block_scan<kWaves>(__popc(eq), sh.wave_sums, &eq_total) + eq_before;
        uint32_t take = gt;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if ((eq >> i) & 1u) {
                if (eq_rank < need) take |= 1u << i;
                ++eq_rank;
            }
        }
        int take_total;
        int pos = block_scan<kWaves>(__popc(take), sh.wave_sums, &take_total) + out_before;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
            if (((take >> i) & 1u) && pos < m) dst[pos++] = src.i(j0 + i);
        eq_before += eq_total;
        out_before += take_total;
    }
}

template <int kWaves, class Src>
__device__ __noinline__ void select_and_emit(SelectShared<kWaves> &sh, const Src &src, int n, int bin, int above,
                                             int m, int32_t *dst)
{
    select_and_emit_inline<kWaves>(sh, src, n, bin, above, m, dst);
}

}  // namespace topk
}  // namespace sa
