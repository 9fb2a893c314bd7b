// Acceptance rate between a dense and a sparse next-token distribution, and its lower-tail
// statistic per bin of positions, on gfx950.
//
// "Sparrow: Sparse Rollout for Stable and Efficient Long-context RL of Large Language Models",
// section 3.1: the mismatch of a sparse rollout with the dense policy is measured per token by
// the acceptance rate alpha = E_{x~q}[min(p(x)/q(x), 1)] = sum_x min(p(x), q(x)) of the two
// next-token distributions p, q (softmax of the logit rows), and summarised per bin of 2K
// positions by a low percentile (the 5th) of the per-token values.
//
//  * acceptance_once_kernel (with a workspace): each logit read once.  A token's rows are split over a
//    group of co-resident workgroups that hold their chunks in registers and exchange the chunks'
//    normalisers through device memory; see the section below.  HBM-bound: 8 bytes per vocabulary entry.
//  * acceptance_rate_kernel (without one): 1024-thread workgroups, two per CU, each taking tokens in turn.
//    Pass 1 streams both logit rows (16-byte loads) keeping an online (max, sum of exp) per thread for
//    each row, reduced over the workgroup; pass 2 streams them again, in reverse order so that the part
//    read last is still in the caches, and sums min(p, q): 16 bytes per vocabulary entry.
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

// ---- each logit read once -------------------------------------------------------------------
// A token's two rows are cut into G consecutive chunks, one per workgroup of a group; the group's G
// workgroups (one per CU, all resident together) take the same tokens in turn.  A workgroup holds its
// chunk of both rows in registers: waves 1..11 (the data waves) hold kA1Per float4 of each row per lane,
// wave 0 exchanges normalisers with the group.  Per token a data wave reduces its lanes to (max, sum of
// exp) per row, keeping exp2(x - lane max) of every entry in place; wave 0 merges the data waves' states
// and publishes the chunk's as one 64-bit word per row (the max's bits low, the sum's high), written and
// polled with relaxed device-scope atomics -- a word is its own flag (an unpublished word has an all-ones
// max, a NaN no reduction produces), so no fence orders it against other data; it waits for the group's
// 2 G words and merges them in chunk order, so every member gets the same normalisers bit for bit.  A
// data wave then sums its entries' min(p, q) (one multiply each: exp2(x - M) = exp2(x - m) exp2(m - M))
// and stores one partial per (token, chunk, wave), which acceptance_sum_kernel adds in that order.
// Wave 0 and the data waves meet only through LDS counters, so the device-wide exchange of token t's
// normalisers proceeds while the data waves load token t + 2 and reduce token t + 1 (three register
// buffers).  Every wait is bounded: each polling lane has kAccSpin device polls for the whole launch
// (about 0.1 s; once spent, a word still unpublished counts as an empty chunk and SA_DEVERR_SYNC is
// flagged -- only if some member could not be scheduled), and each wave kLdsSpin LDS polls for the launch.
constexpr int kA1Threads = 768;
constexpr int kA1Waves = kA1Threads / kWave;
constexpr int kA1DataWaves = kA1Waves - 1;
constexpr int kA1Data = kA1Threads - kWave;              // data lanes: waves 1 .. 11
constexpr int kA1Per = 5;                                 // float4 of each row per data lane and token
constexpr int64_t kA1Chunk = (int64_t)kA1Data * kA1Per;  // float4 of each row per workgroup (3520)
constexpr int kA1MaxGroup = kWave / 2;                    // 2 G words polled by one wave's lanes
constexpr int kA1Slots = 4;                               // normaliser slots (tokens) in LDS
constexpr uint64_t kAccEmpty = ~0ull;
constexpr int kAccSpin = 1 << 16;
constexpr int kLdsSpin = 1 << 24;

__device__ __forceinline__ float max4(float4 v) { return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)); }

__global__ void acceptance_fill_kernel(uint64_t *__restrict__ states, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        states[i] = kAccEmpty;
}

template <int N>
using Rows = float4[N];

// an LDS counter read that the compiler neither caches nor reorders
__device__ __forceinline__ int lds_get(const int *c) { return __hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); }

__global__ __launch_bounds__(kA1Threads, 1) void acceptance_once_kernel(
    const float4 *__restrict__ lp, const float4 *__restrict__ lq, int64_t V4, int64_t ld4, int64_t T, int G,
    int64_t C4, int n_groups, uint64_t *__restrict__ states, float *__restrict__ part, uint32_t *err)
{
    __shared__ float sh_st[2][kA1Waves][4];     // per token parity and data wave: (mp, sp, mq, sq)
    __shared__ float sh_tot[kA1Slots][4];       // per token slot: normalisers (MP, SP, MQ, SQ)
    __shared__ uint64_t sh_words[2 * kA1MaxGroup];
    __shared__ int sh_reduced[2];                // data-wave reductions done, per token parity (sh_st slot)
    __shared__ int sh_ready;                     // tokens whose normalisers are in sh_tot
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int gi = blockIdx.x / G, g = blockIdx.x % G;
    if (gi >= n_groups) return;
    const int64_t c0 = (int64_t)g * C4, c1 = c0 + C4 < V4 ? c0 + C4 : V4;  // this chunk: float4 c0 .. c1 - 1
    const float lowest = -3.402823466e38f;
    auto tok = [&](int64_t r) { return gi + r * n_groups; };  // the group's r-th token
    if (tok(0) >= T) return;
    if (tid == 0) {
        sh_reduced[0] = 0;
        sh_reduced[1] = 0;
        sh_ready = 0;
    }
    __syncthreads();  // the only barrier: the counters are set

    if (wave == 0) {
        int polls = kAccSpin;  // this lane's device polls left
        int spins = kLdsSpin;  // LDS polls left
        for (int64_t r = 0; tok(r) < T; ++r) {
            const int64_t t = tok(r);
            // every data wave has reduced token r: the count of its parity slot reaches 11 (r / 2 + 1) (a wave
            // reduces token r + 2 only after token r's normalisers are ready, so the count never runs ahead)
            while (lds_get(&sh_reduced[r & 1]) < kA1DataWaves * (int)(r / 2 + 1) && spins > 0) {
                --spins;
                __builtin_amdgcn_s_sleep(1);
            }
            uint64_t *const words = states + 2 * (t * G);
            if (lane == 0) {  // the chunk's states, merged over the data waves and published
                const float(*st)[4] = sh_st[r & 1];
                float mp = st[1][0], sp = st[1][1], mq = st[1][2], sq = st[1][3];
                for (int w = 2; w < kA1Waves; ++w) {
                    merge_state(mp, sp, st[w][0], st[w][1]);
                    merge_state(mq, sq, st[w][2], st[w][3]);
                }
                const uint64_t wp = ((uint64_t)__float_as_uint(sp) << 32) | __float_as_uint(mp);
                const uint64_t wq = ((uint64_t)__float_as_uint(sq) << 32) | __float_as_uint(mq);
                __hip_atomic_store(words + 2 * g, wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(words + 2 * g + 1, wq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (lane < 2 * G) {  // lane 2 h + q waits for chunk h's state of row q
                uint64_t v = __hip_atomic_load(words + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                while (v == kAccEmpty && polls > 0) {
                    --polls;
                    __builtin_amdgcn_s_sleep(1);
                    v = __hip_atomic_load(words + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (v == kAccEmpty) {
                    flag_error(err, SA_DEVERR_SYNC);
                    v = (uint64_t)__float_as_uint(lowest);  // (lowest, 0): the chunk counts as empty
                }
                sh_words[lane] = v;
            }
            if (lane == 0) {  // merged in chunk order
                float MP = lowest, SP = 0.f, MQ = lowest, SQ = 0.f;
                for (int h = 0; h < G; ++h) {
                    const uint64_t wp = sh_words[2 * h], wq = sh_words[2 * h + 1];
                    merge_state(MP, SP, __uint_as_float((uint32_t)wp), __uint_as_float((uint32_t)(wp >> 32)));
                    merge_state(MQ, SQ, __uint_as_float((uint32_t)wq), __uint_as_float((uint32_t)(wq >> 32)));
                }
                float *tot = sh_tot[r % kA1Slots];
                tot[0] = MP;
                tot[1] = SP;
                tot[2] = MQ;
                tot[3] = SQ;
                __hip_atomic_store(&sh_ready, (int)(r + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        if (spins == 0) flag_error(err, SA_DEVERR_SYNC);
        return;
    }

    // ---- data waves ----
    const int dl = tid - kWave;
    bool valid[kA1Per];
    uint32_t off[kA1Per];  // lane offsets of the chunk's float4 (lanes past it read its last one, unused)
#pragma unroll
    for (int j = 0; j < kA1Per; ++j) {
        const int64_t i = c0 + dl + (int64_t)kA1Data * j;
        valid[j] = i < c1;
        off[j] = (uint32_t)(16 * (i < c1 ? i : c1 - 1));
    }
    // token t's chunk into (a, b) from uniform row bases (a token past the end reads the last one, unused)
    auto load = [&](int64_t t, Rows<kA1Per> &a, Rows<kA1Per> &b) {
        const int64_t tc = t < T ? t : T - 1;
        const unsigned char *rp = reinterpret_cast<const unsigned char *>(lp + tc * ld4);
        const unsigned char *rq = reinterpret_cast<const unsigned char *>(lq + tc * ld4);
#pragma unroll
        for (int j = 0; j < kA1Per; ++j) {
            uint32_t o = off[j];
            asm volatile("" : "+v"(o));  // kept 32-bit: a uniform base and a lane offset per load
            a[j] = *reinterpret_cast<const float4 *>(rp + o);
            b[j] = *reinterpret_cast<const float4 *>(rq + o);
        }
    };
    // token r's chunk: this wave's (max, sum of exp2) per row into sh_st[r & 1]; the buffer keeps
    // exp2(x - m) of every entry (x = logit * log2 e, m = the lane's maximum, returned in m[0], m[1])
    auto reduce = [&](int64_t r, Rows<kA1Per> &a, Rows<kA1Per> &b, float (&m)[2]) {
        float mp = lowest, mq = lowest;
#pragma unroll
        for (int j = 0; j < kA1Per; ++j)
            if (valid[j]) {
                mp = fmaxf(mp, max4(a[j]) * kLog2e);
                mq = fmaxf(mq, max4(b[j]) * kLog2e);
            }
        float sp = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < kA1Per; ++j) {
            float4 &x = a[j], &y = b[j];
            x.x = exp2_fast(x.x * kLog2e - mp);
            x.y = exp2_fast(x.y * kLog2e - mp);
            x.z = exp2_fast(x.z * kLog2e - mp);
            x.w = exp2_fast(x.w * kLog2e - mp);
            y.x = exp2_fast(y.x * kLog2e - mq);
            y.y = exp2_fast(y.y * kLog2e - mq);
            y.z = exp2_fast(y.z * kLog2e - mq);
            y.w = exp2_fast(y.w * kLog2e - mq);
            if (valid[j]) {
                sp += (x.x + x.y) + (x.z + x.w);
                sq += (y.x + y.y) + (y.z + y.w);
            }
        }
        m[0] = mp;
        m[1] = mq;
        for (int o = kWave / 2; o > 0; o >>= 1) {
            merge_state(mp, sp, __shfl_xor(mp, o), __shfl_xor(sp, o));
            merge_state(mq, sq, __shfl_xor(mq, o), __shfl_xor(sq, o));
        }
        if (lane == 0) {
            float *st = sh_st[r & 1][wave];
            st[0] = mp;
            st[1] = sp;
            st[2] = mq;
            st[3] = sq;
            __hip_atomic_fetch_add(&sh_reduced[r & 1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    };
    int spins = kLdsSpin;
    // token r's minima once its normalisers are ready; one partial per (token, chunk, data wave)
    auto sum = [&](int64_t r, const Rows<kA1Per> &a, const Rows<kA1Per> &b, const float (&m)[2]) {
        while (lds_get(&sh_ready) <= (int)r && spins > 0) {
            --spins;
            __builtin_amdgcn_s_sleep(1);
        }
        const float *tot = sh_tot[r % kA1Slots];
        const float fp = exp2_fast(m[0] - tot[0]) / tot[1], fq = exp2_fast(m[1] - tot[2]) / tot[3];
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kA1Per; ++j)
            if (valid[j]) {
                acc += fminf(a[j].x * fp, b[j].x * fq);
                acc += fminf(a[j].y * fp, b[j].y * fq);
                acc += fminf(a[j].z * fp, b[j].z * fq);
                acc += fminf(a[j].w * fp, b[j].w * fq);
            }
        for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) part[(tok(r) * G + g) * kA1DataWaves + (wave - 1)] = acc;
    };
    // step r: token r + 2's loads out, token r + 1 reduced, token r summed.  A token is reduced two
    // steps before its slot of sh_tot is written again (kA1Slots > 2), and sh_st[r & 1] is rewritten
    // for token r + 2 only after token r's normalisers are ready, i.e. after wave 0 has read it.
    Rows<kA1Per> a0, b0, a1, b1, a2, b2;
    float m0[2], m1[2], m2[2];
    load(tok(0), a0, b0);
    load(tok(1), a1, b1);
    reduce(0, a0, b0, m0);
    for (int64_t r = 0;; r += 3) {
        load(tok(r + 2), a2, b2);
        __builtin_amdgcn_sched_barrier(0);
        if (tok(r + 1) < T) reduce(r + 1, a1, b1, m1);
        __builtin_amdgcn_sched_barrier(0);
        sum(r, a0, b0, m0);
        if (tok(r + 1) >= T) break;
        load(tok(r + 3), a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        if (tok(r + 2) < T) reduce(r + 2, a2, b2, m2);
        __builtin_amdgcn_sched_barrier(0);
        sum(r + 1, a1, b1, m1);
        if (tok(r + 2) >= T) break;
        load(tok(r + 4), a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        if (tok(r + 3) < T) reduce(r + 3, a0, b0, m0);
        __builtin_amdgcn_sched_barrier(0);
        sum(r + 2, a2, b2, m2);
        if (tok(r + 3) >= T) break;
    }
    if (spins == 0) flag_error(err, SA_DEVERR_SYNC);
}

// alpha[t] = the sum of token t's n partials (G chunks x kA1DataWaves waves), one wave per token: lane l adds
// partials l, l + 64, ... in order, then a fixed butterfly over the lanes, so the result is the same on every call.
__global__ void acceptance_sum_kernel(const float *__restrict__ part, int n, int64_t T, float *__restrict__ alpha)
{
    const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = lane_id();
    if (t >= T) return;
    float acc = 0.f;
    for (int h = lane; h < n; h += kWave) acc += part[t * n + h];
    for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) alpha[t] = acc;
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

int acceptance_group(const sa_handle_s &h, int64_t V)
{
    if (V % 4 != 0) return 0;
    const int64_t G = (V / 4 + kA1Chunk - 1) / kA1Chunk;
    return G <= kA1MaxGroup && G <= h.n_cu ? (int)G : 0;
}

size_t acceptance_workspace(const sa_handle_s &h, int64_t T, int64_t V)
{
    const int G = acceptance_group(h, V);
    if (G == 0) return 0;
    // 2 G state words, then G x (data waves) partial sums, per token
    return (size_t)T * G * (2 * sizeof(uint64_t)) + (size_t)T * G * kA1DataWaves * sizeof(float);
}

hipError_t launch_acceptance_rate(sa_handle_s &h, const float *lp, const float *lq, int64_t T, int64_t V, int64_t ld,
                                  float *alpha, void *ws, hipStream_t st)
{
    const bool vec = V % 4 == 0 && ld % 4 == 0 && (reinterpret_cast<uintptr_t>(lp) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(lq) & 15u) == 0;
    const int G = vec && ws ? acceptance_group(h, V) : 0;
    if (G > 0) {
        uint64_t *states = static_cast<uint64_t *>(ws);
        float *part = reinterpret_cast<float *>(states + (size_t)T * G * 2);
        const int n_groups = h.n_cu / G;
        const int64_t V4 = V / 4, C4 = (V4 + G - 1) / G;
        {
            KernelTimer timer(h, SA_KERNEL_ACCEPT, st);
            const int64_t n = T * G * 2;
            const int64_t blocks = (n + 255) / 256 < 4 * (int64_t)h.n_cu ? (n + 255) / 256 : 4 * (int64_t)h.n_cu;
            hipLaunchKernelGGL(acceptance_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, states, n);
        }
        {
            KernelTimer timer(h, SA_KERNEL_ACCEPT, st);
            hipLaunchKernelGGL(acceptance_once_kernel, dim3((unsigned)(n_groups * G)), dim3(kA1Threads), 0, st,
                               reinterpret_cast<const float4 *>(lp), reinterpret_cast<const float4 *>(lq), V4, ld / 4,
                               T, G, C4, n_groups, states, part, h.d_err);
        }
        KernelTimer timer(h, SA_KERNEL_ACCEPT, st);
        hipLaunchKernelGGL(acceptance_sum_kernel, dim3((unsigned)((T + 3) / 4)), dim3(4 * kWave), 0, st, part,
                           G * kA1DataWaves, T, alpha);
        return hipGetLastError();
    }
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
