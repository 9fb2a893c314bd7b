// Acceptance rate between a dense and a sparse next-token distribution, and its lower-tail
// statistic per bin of positions, on gfx950.
//
// "Sparrow: Sparse Rollout for Stable and Efficient Long-context RL of Large Language Models",
// section 3.1: the mismatch of a sparse rollout with the dense policy is measured per token by
// the acceptance rate alpha = E_{x~q}[min(p(x)/q(x), 1)] = sum_x min(p(x), q(x)) of the two
// next-token distributions p, q (softmax of the logit rows), and summarised per bin of 2K
// positions by a low percentile (the 5th) of the per-token values.
//
//  * acceptance_rate_kernel: 1024-thread workgroups, two per CU, each taking tokens in turn (more loads
//    in flight per workgroup than one small workgroup per token: 12 % faster).  Pass 1 streams both logit rows
//    once (16-byte loads) keeping an online (max, sum of exp) per thread for each row, reduced
//    over the workgroup; pass 2 streams them again, in reverse order so that the part read last
//    is still in the caches, and sums min(p, q).  HBM-bound: 8 bytes per vocabulary entry.
//  * bin_stats_kernel: one workgroup per bin.  The count and the (double) sum of the bin's values
//    from one scan of the tokens, which also stages their order keys in LDS (up to 8192), then the two
//    order statistics around the percentile, each found exactly by an MSD radix select over the order
//    keys (four 8-bit passes with a 256-bin LDS histogram, over the staged keys, or over the tokens
//    again for a larger bin), and the linear interpolation between them.
#include <math.h>

#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

namespace {

constexpr int kAccThreads = 1024;
constexpr int kAccWaves = kAccThreads / kWave;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge an online softmax state (m, s): s = sum exp(x - m), in the log2 domain.
__device__ __forceinline__ void merge_state(float &m, float &s, float m2, float s2)
{
    const float mn = fmaxf(m, m2);
    s = (m == mn ? s : s * exp2_fast(m - mn)) + (m2 == mn ? s2 : s2 * exp2_fast(m2 - mn));
    m = mn;
}

__device__ __forceinline__ void add_value(float &m, float &s, float x)
{
    if (x > m) {
        s = s * exp2_fast(m - x) + 1.f;
        m = x;
    } else {
        s += exp2_fast(x - m);
    }
}

// Workgroup-wide merge of (m, s) states; every thread gets the result.
__device__ __forceinline__ void reduce_state(float &m, float &s, float (*sh)[2])
{
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
        merge_state(m, s, m2, s2);
    }
    const int wave = threadIdx.x / kWave;
    __syncthreads();
    if (lane_id() == 0) {
        sh[wave][0] = m;
        sh[wave][1] = s;
    }
    __syncthreads();
    m = sh[0][0];
    s = sh[0][1];
    for (int i = 1; i < kAccWaves; ++i) merge_state(m, s, sh[i][0], sh[i][1]);
}

__device__ __forceinline__ float block_sum(float v, float *sh)
{
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x / kWave;
    __syncthreads();
    if (lane_id() == 0) sh[wave] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < kAccWaves; ++i) t += sh[i];
    return t;
}

// vec: rows are 16-byte aligned and V % 4 == 0 (float4 loads); otherwise one float at a time.
template <bool vec>
__global__ __launch_bounds__(kAccThreads) void acceptance_rate_kernel(const float *__restrict__ lp,
                                                                      const float *__restrict__ lq, int64_t V,
                                                                      int64_t ld, float *__restrict__ alpha, int64_t T)
{
    __shared__ float shs[kAccWaves][2];
    __shared__ float shr[kAccWaves];
    const int tid = threadIdx.x;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const float *rp = lp + t * ld, *rq = lq + t * ld;
        // the running maxima start at the lowest finite float, so a -inf logit (a masked entry) adds
        // exp2(-inf) = 0 and never meets another -inf in a difference
        const float lowest = -3.402823466e38f;

        // pass 1: max and sum of exp per row (log2 domain)
        float mp = lowest, sp = 0.f, mq = lowest, sq = 0.f;
        if (vec) {
            const int64_t n4 = V / 4;
            for (int64_t i = tid; i < n4; i += kAccThreads) {
                const float4 a = reinterpret_cast<const float4 *>(rp)[i];
                const float4 b = reinterpret_cast<const float4 *>(rq)[i];
                add_value(mp, sp, a.x * kLog2e);
                add_value(mp, sp, a.y * kLog2e);
                add_value(mp, sp, a.z * kLog2e);
                add_value(mp, sp, a.w * kLog2e);
                add_value(mq, sq, b.x * kLog2e);
                add_value(mq, sq, b.y * kLog2e);
                add_value(mq, sq, b.z * kLog2e);
                add_value(mq, sq, b.w * kLog2e);
            }
        } else {
            for (int64_t i = tid; i < V; i += kAccThreads) {
                add_value(mp, sp, rp[i] * kLog2e);
                add_value(mq, sq, rq[i] * kLog2e);
            }
        }
        reduce_state(mp, sp, shs);
        reduce_state(mq, sq, shs);
        const float ip = 1.f / sp, iq = 1.f / sq;

        // pass 2: sum of min(p, q), last-read data first
        float acc = 0.f;
        if (vec) {
            const int64_t n4 = V / 4;
            const int64_t top = (n4 + kAccThreads - 1) / kAccThreads * kAccThreads;
            for (int64_t base = top - kAccThreads; base >= 0; base -= kAccThreads) {
                const int64_t i = base + tid;
                if (i < n4) {
                    const float4 a = reinterpret_cast<const float4 *>(rp)[i];
                    const float4 b = reinterpret_cast<const float4 *>(rq)[i];
                    acc += fminf(exp2_fast(a.x * kLog2e - mp) * ip, exp2_fast(b.x * kLog2e - mq) * iq);
                    acc += fminf(exp2_fast(a.y * kLog2e - mp) * ip, exp2_fast(b.y * kLog2e - mq) * iq);
                    acc += fminf(exp2_fast(a.z * kLog2e - mp) * ip, exp2_fast(b.z * kLog2e - mq) * iq);
                    acc += fminf(exp2_fast(a.w * kLog2e - mp) * ip, exp2_fast(b.w * kLog2e - mq) * iq);
                }
            }
        } else {
            for (int64_t i = tid; i < V; i += kAccThreads)
                acc += fminf(exp2_fast(rp[i] * kLog2e - mp) * ip, exp2_fast(rq[i] * kLog2e - mq) * iq);
        }
        acc = block_sum(acc, shr);
        if (tid == 0) alpha[t] = acc;
    }
}

// The inverse of order_key.
__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

constexpr int kBinThreads = 256;

__device__ __forceinline__ int64_t bin_of(int32_t p, int32_t bin_size) { return p >= 0 ? p / bin_size : -1; }

// The value of rank r (0-based, ascending) among the bin's values: four 8-bit MSD passes.
__device__ float rank_value(const float *__restrict__ alpha, const int32_t *__restrict__ pos, int64_t T,
                            int32_t bin_size, int64_t bin, int64_t r, uint32_t *hist, uint32_t *sh_digit,
                            int64_t *sh_rank)
{
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int64_t t = tid; t < T; t += kBinThreads) {
            if (bin_of(pos[t], bin_size) != bin) continue;
            const uint32_t k = order_key(alpha[t]);
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            int64_t c = 0;
            for (int d = 0; d < 256; ++d) {
                if (c + hist[d] > r) {
                    *sh_digit = (uint32_t)d;
                    *sh_rank = r - c;
                    break;
                }
                c += hist[d];
            }
        }
        __syncthreads();
        prefix |= *sh_digit << shift;
        mask |= 255u << shift;
        r = *sh_rank;
        __syncthreads();
    }
    return key_value(prefix);
}

// The same from the bin's n <= kBinCap order keys staged in LDS: four 8-bit MSD passes over LDS, each digit found
// by one wave's prefix scan of the 256-bin histogram.
constexpr int kBinCap = 8192;
__device__ float rank_value_lds(const uint32_t *keys, int n, int64_t r, uint32_t *hist, uint32_t *sh_digit,
                                int64_t *sh_rank)
{
    const int tid = threadIdx.x, lane = lane_id();
    uint32_t prefix = 0, mask = 0;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kBinThreads) {
            const uint32_t k = keys[i];
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l holds digits 4 l .. 4 l + 3; the lane whose counts span rank r names the digit
            uint32_t c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = hist[4 * lane + j];
            const uint32_t own = c[0] + c[1] + c[2] + c[3];
            uint32_t incl = own;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t v = __shfl_up(incl, off);
                if (lane >= off) incl += v;
            }
            int64_t below = (int64_t)(incl - own);
            if (below <= r && r < (int64_t)incl) {
                int j = 0;
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    if (j == q && below + c[q] <= r) {
                        below += c[q];
                        j = q + 1;
                    }
                }
                *sh_digit = (uint32_t)(4 * lane + j);
                *sh_rank = r - below;
            }
        }
        __syncthreads();
        prefix |= *sh_digit << shift;
        mask |= 255u << shift;
        r = *sh_rank;
        __syncthreads();
    }
    return key_value(prefix);
}

__global__ __launch_bounds__(kBinThreads) void bin_stats_kernel(const float *__restrict__ alpha,
                                                                const int32_t *__restrict__ pos, int64_t T,
                                                                int32_t bin_size, double percentile,
                                                                int32_t *__restrict__ count, float *__restrict__ mean,
                                                                float *__restrict__ pct)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_digit;
    __shared__ int64_t sh_rank;
    __shared__ double sh_sum[kBinThreads / kWave];
    __shared__ int64_t sh_cnt[kBinThreads / kWave];
    __shared__ uint32_t keys[kBinCap];  // the bin's order keys, in no particular order (up to kBinCap)
    __shared__ uint32_t sh_staged;
    const int64_t bin = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid == 0) sh_staged = 0;
    __syncthreads();

    double sum = 0.0;
    int64_t n = 0;
    for (int64_t t = tid; t < T; t += kBinThreads) {
        if (bin_of(pos[t], bin_size) != bin) continue;
        const float a = alpha[t];
        sum += (double)a;
        ++n;
        const uint32_t slot = atomicAdd(&sh_staged, 1u);
        if (slot < (uint32_t)kBinCap) keys[slot] = order_key(a);
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        sum += __shfl_xor(sum, off);
        n += __shfl_xor(n, off);
    }
    if (lane_id() == 0) {
        sh_sum[tid / kWave] = sum;
        sh_cnt[tid / kWave] = n;
    }
    __syncthreads();
    sum = 0.0;
    n = 0;
    for (int i = 0; i < kBinThreads / kWave; ++i) {
        sum += sh_sum[i];
        n += sh_cnt[i];
    }
    if (n == 0) {
        if (tid == 0) {
            count[bin] = 0;
            mean[bin] = __builtin_nanf("");
            pct[bin] = __builtin_nanf("");
        }
        return;
    }
    const double h = (double)(n - 1) * percentile / 100.0;
    const int64_t lo = (int64_t)floor(h);
    const int64_t hi = lo + 1 < n ? lo + 1 : n - 1;
    float x_lo, x_hi;
    if (n <= kBinCap) {  // all of the bin's values are in LDS
        x_lo = rank_value_lds(keys, (int)n, lo, hist, &sh_digit, &sh_rank);
        x_hi = hi == lo ? x_lo : rank_value_lds(keys, (int)n, hi, hist, &sh_digit, &sh_rank);
    } else {
        x_lo = rank_value(alpha, pos, T, bin_size, bin, lo, hist, &sh_digit, &sh_rank);
        x_hi = hi == lo ? x_lo : rank_value(alpha, pos, T, bin_size, bin, hi, hist, &sh_digit, &sh_rank);
    }
    if (tid == 0) {
        count[bin] = (int32_t)n;
        mean[bin] = (float)(sum / (double)n);
        pct[bin] = (float)((double)x_lo + (h - (double)lo) * ((double)x_hi - (double)x_lo));
    }
}

}  // namespace

hipError_t launch_acceptance_rate(sa_handle_s &h, const float *lp, const float *lq, int64_t T, int64_t V, int64_t ld,
                                  float *alpha, hipStream_t st)
{
    const bool vec = V % 4 == 0 && ld % 4 == 0 && (reinterpret_cast<uintptr_t>(lp) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(lq) & 15u) == 0;
    KernelTimer timer(h, SA_KERNEL_ACCEPT, st);
    const int64_t grid = T < 2 * (int64_t)h.n_cu ? T : 2 * (int64_t)h.n_cu;  // two workgroups per CU
    if (vec)
        hipLaunchKernelGGL(acceptance_rate_kernel<true>, dim3((unsigned)grid), dim3(kAccThreads), 0, st, lp, lq, V, ld,
                           alpha, T);
    else
        hipLaunchKernelGGL(acceptance_rate_kernel<false>, dim3((unsigned)grid), dim3(kAccThreads), 0, st, lp, lq, V, ld,
                           alpha, T);
    return hipGetLastError();
}

hipError_t launch_bin_stats(sa_handle_s &h, const float *alpha, const int32_t *pos, int64_t T, int32_t bin_size,
                            int32_t n_bins, float percentile, int32_t *count, float *mean, float *pct, hipStream_t st)
{
    KernelTimer timer(h, SA_KERNEL_ACCEPT, st);
    hipLaunchKernelGGL(bin_stats_kernel, dim3((unsigned)n_bins), dim3(kBinThreads), 0, st, alpha, pos, T, bin_size,
                       (double)percentile, count, mean, pct);
    return hipGetLastError();
}

}  // namespace sa
