// Fused prefill indexer + streaming per-query top-k on gfx950.
//
// For every query row t of one sequence: the scores I(t,s) = sum_j w(t,j) ReLU(q(t,j).k(s))
// over the visible keys s <= t ("Sparse Attention and RL Optimization: Three Technical
// Breakthroughs in LLM Post-Training", section 2.2, with the causal look-back rule of the
// section 2.5 pseudocode) and the min(k, t+1) keys of largest score, ties to the lower key
// (section 2.3).  The [L, L] score matrix is never formed.
//
// Design (bf16, H_I = 64 index heads, d_I = 128):
//  * Persistent workgroups of 8 waves pull tiles of 8 query rows from an atomic counter,
//    latest rows (most keys) first.  Wave w owns query row q0 + w for the whole tile: its
//    A operand (64 heads x 128 dims of q, 64 VGPRs) and head weights stay in registers.
//  * Keys stream through LDS in 64-key tiles (16 KB, double-buffered, 16-byte chunks XOR-
//    swizzled so that the MFMA fragment reads are free of bank conflicts).  Per tile each
//    wave issues 32 v_mfma_f32_32x32x16_bf16: heads on M (2 tiles of 32), keys on N (2 tiles
//    of 32), d_I on K.  fp32 accumulation.
//  * Epilogue in registers: each lane holds 16 head rows of one key column per 32x32 tile;
//    ReLU, the weight and the head sum run in-lane, one v_permlane32_swap finishes the head
//    sum and leaves lane l with the score of key tile_base + l.
//  * Streaming top-k: every score bumps a per-row 2048-bin LDS histogram of its order-
//    preserving key's top 11 bits.  From it the wave keeps a running threshold bin: once m
//    scores lie in bins >= b, no score in a lower bin can be selected.  Only scores in bins
//    >= the running threshold are appended (ballot-compacted, in key order) to the row's
//    candidate list in the workspace -- about m (1 + ln(t/m)) of the t+1 scores.
//  * At the end of the tile the final histogram fixes the threshold bin b* exactly.  The
//    candidates in bins >= b* are gathered into LDS (at most kCap; otherwise the list is
//    scanned in global memory), an MSD radix select over the remaining 21 key bits finds the
//    exact m-th key, and an ordered compaction writes the selection in ascending key order.
#include "sa_device.hpp"
#include "sa_internal.hpp"
#include "topk_device.hpp"

namespace sa {

namespace {

constexpr int kH = 64;              // index heads
constexpr int kD = 128;             // index head width
constexpr int kRows = 8;            // query rows per tile = waves per workgroup
constexpr int kThreads = kRows * kWave;
constexpr int kKT = 64;             // keys per LDS tile
constexpr int kHalves = kKT / 32;   // 32-key MFMA column blocks per tile
constexpr int kTileLoads = kKT * 16 / 512;  // 16-byte chunks each thread moves per tile
constexpr int kChunks = kD * 2 / 16;  // 16-byte chunks per key row (16)
constexpr int kRefresh = 8;         // key tiles between running-threshold refreshes
using topk::kBins;
using topk::kBinShift;
using topk::kCap;
using topk::kPerThread;

static_assert(kRows * kBins * 4 == kCap * 8, "the histogram region holds the candidates");

struct Shared {
    uint4 keys[2][kKT * kChunks];        // double-buffered key tiles
    uint32_t region[kRows * kBins];      // 64 KB: histograms, then candidate (key, index)
    topk::SelectShared<kRows> sel;
    int info[kRows][4];                  // per row: b*, count in bins > b*, count in bins >= b*,
                                         // candidate list length
    int tile;
};

// Scheduling pattern of one 32-key half-tile: its 8 B-fragment reads, then the 16 MFMAs
// interleaved with the 64 VALU ops of the previous half-tile's epilogue.
template <int kId>
__device__ __forceinline__ void interleave_half()
{
    __builtin_amdgcn_sched_group_barrier(0x100, 8, kId);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, kId);
#pragma unroll
    for (int i = 0; i < 14; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, kId);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, kId);
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 8, kId);
}

__global__ __launch_bounds__(kThreads, 1) void indexer_topk_prefill_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w, const uint16_t *__restrict__ k_idx,
    int64_t L, int32_t topk, int32_t *__restrict__ idx, uint2 *__restrict__ cands, int64_t cand_ld,
    int32_t *__restrict__ counter, int32_t n_tiles)
{
    __shared__ Shared sh;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    uint2 *my_cands = cands + ((int64_t)blockIdx.x * kRows + wave) * cand_ld;

#pragma unroll 1
    for (;;) {
        if (tid == 0) sh.tile = atomicAdd(counter, 1);
        __syncthreads();
        const int it = sh.tile;
        if (it >= n_tiles) break;
        const int64_t q0 = (int64_t)(n_tiles - 1 - it) * kRows;  // latest rows first
        const int64_t t_last = (q0 + kRows - 1 < L - 1) ? q0 + kRows - 1 : L - 1;
        const int64_t row = q0 + wave;
        const bool row_ok = row < L;
        const int m = row_ok ? (int)((int64_t)topk < row + 1 ? (int64_t)topk : row + 1) : 0;
        const bool selects = row_ok && row + 1 > topk;  // fewer than all visible keys
        int n_cand = 0;                                    // this row's candidate list length

        if (t_last + 1 > topk) {  // some row of the tile needs scores
            for (int i = tid; i < kRows * kBins; i += kThreads) sh.region[i] = 0;

            // A operand and weights of this wave's query row
            bf16x8 a[2][kD / 16];
            float wv[2][16];
            const int64_t qrow = row_ok ? row : L - 1;
            const uint16_t *qr = q_idx + qrow * (int64_t)kH * kD;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int ks = 0; ks < kD / 16; ++ks)
                    a[mt][ks] = as_bf16x8(load16(qr + (32 * mt + lane % 32) * kD + 16 * ks + 8 * (lane / 32)));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int g = 0; g < 16; ++g)
                    wv[mt][g] = w[qrow * kH + 32 * mt + 8 * (g / 4) + 4 * (lane / 32) + g % 4];

            // key tile loader: thread i moves chunks i and i + 512 of the 1024 in a tile;
            // LDS slot (r, j) holds chunk j ^ (r % 16) of key row r
            const int n_kt = (int)(t_last / kKT) + 1;
            auto load_tile = [&](int kt, uint4 (&v)[kTileLoads]) {
#pragma unroll
                for (int u = 0; u < kTileLoads; ++u) {
                    const int c = tid + u * kThreads;
                    const int r = c / kChunks, j = c % kChunks;
                    int64_t s = (int64_t)kt * kKT + r;
                    if (s > t_last) s = t_last;
                    v[u] = load16(k_idx + s * kD + 8 * (j ^ (r % 16)));
                }
            };
            auto store_tile = [&](int buf, const uint4 (&v)[kTileLoads]) {
#pragma unroll
                for (int u = 0; u < kTileLoads; ++u) sh.keys[buf][tid + u * kThreads] = v[u];
            };
            {
                uint4 v[kTileLoads];
                load_tile(0, v);
                store_tile(0, v);
            }
            uint32_t *hist = sh.region + wave * kBins;
            int run_bin = 0;  // running threshold bin: scores in lower bins are dropped

            // Software pipeline over half-tiles of 32 keys: while the MFMAs of half-tile h run,
            // the VALU applies ReLU, the weights and the in-lane head sum to the accumulators of
            // half-tile h - 1.  acc[0] holds the even half-tiles, acc[1] the odd ones; a window
            // of 64 keys shifted by -32 (odd half of tile kt - 1, even half of tile kt) is then
            // finished by one v_permlane32_swap: lane l scores key 64 kt - 32 + l.
            f32x16 acc[2][2];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) acc[st][mt] = f32x16{};

            // all keys of a window go through the histogram; the ones at or above the running
            // threshold bin are appended to the row's candidate list in key order
            auto finish_window = [&](float part_odd, float part_even, int64_t s) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part_odd),
                                                                 __float_as_uint(part_even), false, false);
                const float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                const bool vis = s >= 0 && s <= row;
                const uint32_t key = order_key(score);
                atomicAdd(&hist[key >> kBinShift], vis ? 1u : 0u);
                const bool keep = vis && (int)(key >> kBinShift) >= run_bin;
                const uint64_t ballot = __ballot(keep);
                if (keep) {
                    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
                    my_cands[n_cand + rank] = make_uint2(key, (uint32_t)s);
                }
                n_cand += __popcll(ballot);
            };

#pragma unroll 1
            for (int kt = 0; kt < n_kt; ++kt) {
                __syncthreads();
                uint4 nxt[kTileLoads];
                const bool more = kt + 1 < n_kt;
                if (more) load_tile(kt + 1, nxt);
                if (selects) {
                    const uint4 *kb = sh.keys[kt & 1];
                    float part_odd = 0.f;
#pragma unroll
                    for (int hf = 0; hf < kHalves; ++hf) {
                        const int st = hf & 1;  // accumulator pair of this half-tile
                        // B fragments of half-tile hf: key 32 hf + l % 32, dims 16 ks + 8 (l / 32)
                        bf16x8 b[kD / 16];
#pragma unroll
                        for (int ks = 0; ks < kD / 16; ++ks) {
                            const int r = 32 * hf + lane % 32;
                            const int j = (2 * ks + lane / 32) ^ (r % 16);
                            b[ks] = as_bf16x8(kb[r * kChunks + j]);
                        }
                        // epilogue of the previous half-tile (the other accumulator pair):
                        // register g of lane l is head 32 mt + 8 (g / 4) + 4 (l / 32) + g % 4
                        float p = 0.f;
#pragma unroll
                        for (int g = 0; g < 16; ++g) {
                            p = fmaf(wv[0][g], relu(acc[st ^ 1][0][g]), p);
                            p = fmaf(wv[1][g], relu(acc[st ^ 1][1][g]), p);
                        }
                        acc[st][0] = f32x16{};
                        acc[st][1] = f32x16{};
#pragma unroll
                        for (int ks = 0; ks < kD / 16; ++ks)
#pragma unroll
                            for (int mt = 0; mt < 2; ++mt)
                                acc[st][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][ks], b[ks],
                                                                                      acc[st][mt], 0, 0, 0);
                        // 8 fragment reads, then one MFMA per 4 VALU of the epilogue
                        if (hf == 0) interleave_half<0>();
                        else if (hf == 1) interleave_half<1>();
                        else if (hf == 2) interleave_half<2>();
                        else interleave_half<3>();
                        if (st == 0) {
                            part_odd = p;  // odd half-tile before this one
                        } else {
                            // window: odd half-tile hf - 2 and even half-tile hf - 1
                            finish_window(part_odd, p, (int64_t)kt * kKT + 32 * (hf - 2) + lane);
                        }
                    }
                    if ((kt % kRefresh) == kRefresh - 1 && (int64_t)kt * kKT >= m) {
                        const int b = topk::threshold_bin(hist, m, nullptr, nullptr);
                        if (b > run_bin) run_bin = b;
                    }
                }
                if (more) store_tile((kt + 1) & 1, nxt);
            }
            if (selects) {  // the odd half of the last tile
                float p = 0.f;
#pragma unroll
                for (int g = 0; g < 16; ++g) {
                    p = fmaf(wv[0][g], relu(acc[1][0][g]), p);
                    p = fmaf(wv[1][g], relu(acc[1][1][g]), p);
                }
                finish_window(p, 0.f, (int64_t)n_kt * kKT - 32 + lane);
            }
        }
        // final threshold per row (each wave its own row), then free the histograms
        if (selects) {
            int ab, up;
            const int b = topk::threshold_bin(sh.region + wave * kBins, m, &ab, &up);
            if (lane == 0) {
                sh.info[wave][0] = b;
                sh.info[wave][1] = ab;
                sh.info[wave][2] = up;
            }
        }
        if (lane == 0) sh.info[wave][3] = n_cand;
        __syncthreads();

#pragma unroll 1
        for (int r = 0; r < kRows; ++r) {
            const int64_t rr = q0 + r;
            if (rr >= L) break;
            int32_t *dst = idx + rr * topk;
            if (rr + 1 <= topk) {  // every visible key is selected
                for (int i = tid; i < topk; i += kThreads) dst[i] = i <= rr ? i : -1;
                continue;
            }
            const int mr = topk;
            const int bin = sh.info[r][0], above = sh.info[r][1], upto = sh.info[r][2];
            const uint2 *list = cands + ((int64_t)blockIdx.x * kRows + r) * cand_ld;
            const int nl = sh.info[r][3];
            if (upto <= kCap) {
                // gather the candidates in bins >= bin into LDS, keeping their order
                uint32_t *ck = sh.region;
                int32_t *ci = reinterpret_cast<int32_t *>(sh.region + kCap);
                const uint32_t lo = (uint32_t)bin << kBinShift;
                int out_before = 0;
#pragma unroll 1
                for (int base = 0; base < nl; base += kThreads * kPerThread) {
                    const int j0 = base + tid * kPerThread;
                    uint2 c[kPerThread];
                    uint32_t sel = 0;
#pragma unroll
                    for (int i = 0; i < kPerThread; ++i) {
                        c[i] = j0 + i < nl ? list[j0 + i] : make_uint2(0u, 0u);
                        sel |= (j0 + i < nl && c[i].x >= lo ? 1u : 0u) << i;
                    }
                    int total;
                    int pos = topk::block_scan<kRows>(__popc(sel), sh.sel.wave_sums, &total) + out_before;
#pragma unroll
                    for (int i = 0; i < kPerThread; ++i)
                        if ((sel >> i) & 1u) {
                            ck[pos] = c[i].x;
                            ci[pos] = (int32_t)c[i].y;
                            ++pos;
                        }
                    out_before += total;
                }
                __syncthreads();
                topk::select_and_emit(sh.sel, topk::LdsCands{ck, ci}, upto, bin, above, mr, dst);
            } else {
                topk::select_and_emit(sh.sel, topk::GlobalCands{list}, nl, bin, above, mr, dst);
            }
            for (int i = mr + tid; i < topk; i += kThreads) dst[i] = -1;
            __syncthreads();
        }
    }
}

__global__ void reset_counter_kernel(int32_t *counter) { *counter = 0; }

}  // namespace

size_t prefill_topk_workspace(const sa_handle_s &h, int64_t L)
{
    const int64_t n_tiles = (L + kRows - 1) / kRows;
    const int64_t slots = n_tiles < h.n_cu ? n_tiles : h.n_cu;
    const int64_t ld = (L + 63) / 64 * 64;
    return 256 + (size_t)slots * kRows * (size_t)ld * sizeof(uint2);
}

hipError_t launch_prefill_topk(sa_handle_s &h, const void *q_idx, const float *w, const void *k_idx,
                               int64_t L, int32_t topk, int32_t *idx, void *ws, hipStream_t st)
{
    const int64_t n_tiles = (L + kRows - 1) / kRows;
    const int64_t slots = n_tiles < h.n_cu ? n_tiles : h.n_cu;
    const int64_t ld = (L + 63) / 64 * 64;
    int32_t *counter = reinterpret_cast<int32_t *>(ws);
    uint2 *cands = reinterpret_cast<uint2 *>(reinterpret_cast<char *>(ws) + 256);
    hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(1), 0, st, counter);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    KernelTimer timer(h, SA_KERNEL_INDEXER, st);
    hipLaunchKernelGGL(indexer_topk_prefill_kernel, dim3((unsigned)slots), dim3(kThreads), 0, st,
                       reinterpret_cast<const uint16_t *>(q_idx), w, reinterpret_cast<const uint16_t *>(k_idx),
                       L, topk, idx, cands, ld, counter, (int32_t)n_tiles);
    return hipGetLastError();
}

}  // namespace sa
