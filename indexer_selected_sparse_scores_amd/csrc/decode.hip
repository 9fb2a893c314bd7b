// Paged decode: indexer scores over the whole cached context and the per-sequence top-k, on
// gfx950.
//
// One new token per sequence attends to the k_b most relevant of its n_b cached tokens
// ("Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and
// Verifiable Synthetic Data", section 2.3: the indexer scores every cached token, and only the
// selected KV entries are read, through the paged cache).  The score is
// I(s) = sum_j w(j) ReLU(q(j).k(s)) ("Sparse Attention and RL Optimization: Three Technical
// Breakthroughs in LLM Post-Training", section 2.2); selection keeps the largest scores,
// ties to the lower token index (section 2.3).
//
// Fast path (bf16, H_I = 64, d_I = 128, 64-token pages), two kernels after a histogram reset:
//  * indexer_decode_kernel: grid (1024-key blocks, sequences).  Each wave streams 4 pages of
//    index keys straight into v_mfma_f32_32x32x16_bf16 B fragments (next half-page in flight
//    while the current one is multiplied; q fragments and head weights are read from LDS, which
//    leaves room for four waves per SIMD and so more key bytes in flight), applies
//    ReLU / weights / head sum in registers, counts the fp32 scores in a 2048-bin LDS histogram
//    that is added to the sequence's histogram in global memory, and gathers each wave's 256
//    scores in LDS for one store at its end.  The scan over index keys is the HBM-bound part
//    of decode (256 bytes per cached token).
//  * decode_topk_kernel: 1024-thread workgroups, one per 32768-token chunk of a sequence.  From
//    the histogram, the bin b* holding the k_b-th largest score; every score of the chunk in
//    bins >= b* is appended, in token order, to a candidate list in LDS (the scores stream in
//    coalesced rounds).  The chunks' lists meet in the sequence's list in global memory; the
//    last chunk to finish gathers them in chunk order, takes the exact k_b-th key by an MSD
//    radix select and writes the selection in ascending order.  A sequence whose candidates
//    exceed the list is selected from its full score row.
#include "sa_device.hpp"
#include "sa_internal.hpp"
#include "topk_device.hpp"

namespace sa {

namespace {

constexpr int kH = 64;                 // index heads
constexpr int kD = 128;                // index head width
constexpr int kPage = 64;              // tokens per page
constexpr int kIdxThreads = 256;       // indexer workgroup (4 waves)
constexpr int kPagesPerWave = 4;
constexpr int kKeysPerBlock = kPage * kPagesPerWave * (kIdxThreads / kWave);  // 1024
constexpr int kTopkWaves = 16;                      // selection workgroup: one per sequence
constexpr int kTopkThreads = kTopkWaves * kWave;
constexpr int kSubRounds = 4;                       // float4 loads per thread per round
constexpr int kRoundScores = kSubRounds * 4 * kTopkThreads;  // 16384 scores per round
constexpr int kTopkChunk = 2 * kRoundScores;        // tokens per selection workgroup
static_assert(kSubRounds * kTopkWaves == kWave, "one (sub-round, wave) count per lane");
using topk::kBins;
using topk::kBinShift;
using topk::kCap;

__device__ __forceinline__ bool decode_row_ok(const int32_t *ctx_len, const int32_t *topk_b, int32_t max_ctx,
                                              int32_t max_topk, int64_t b, int64_t *n, int64_t *m)
{
    *n = ctx_len[b];
    const int64_t k = topk_b[b];
    if (*n < 1 || *n > max_ctx || k < 1 || k > max_topk) return false;
    *m = k < *n ? k : *n;
    return true;
}

// clears the histograms and the selection's sync words (a kernel, not a memset, so that a captured graph
// replays it)
__global__ void decode_reset_kernel(uint32_t *hist, uint32_t *sync, int64_t B)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < B * kBins) hist[i] = 0;
    if (i < 2 * B) sync[i] = 0;
}

// q (as MFMA A fragments) and the head weights of the workgroup's sequence live in LDS, so a wave holds
// only its key fragments and accumulators and four waves fit on a SIMD: more key bytes in flight.
struct DecodeIdxShared {
    uint4 qf[2 * (kD / 16) * kWave];  // fragment (mt, ks) of lane l at (8 mt + ks) * 64 + l: 16 KB
    float4 wq[kH / 4];                // the 64 head weights
    uint32_t hist[kBins];
    float4 sc[kIdxThreads / kWave][kPagesPerWave * kPage / 4];  // each wave's 256 scores, stored at the end
};

__global__ __launch_bounds__(kIdxThreads, 4) void indexer_decode_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w, const uint16_t *__restrict__ kidx_pages,
    int64_t n_pages, const int32_t *__restrict__ block_table, int32_t max_blocks,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ row_seq, int32_t max_ctx,
    float *__restrict__ scores, int64_t ld, uint32_t *__restrict__ hist_g, uint32_t *__restrict__ pmax_g,
    int64_t pmax_ld, uint32_t *err)
{
    __shared__ DecodeIdxShared sh;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int64_t b = blockIdx.y;  // query row: its q, weights, context length and outputs
    const int64_t n = ctx_len[b];
    if (n < 1 || n > max_ctx) {
        if (tid == 0 && blockIdx.x == 0) flag_error(err, SA_DEVERR_CTX_LEN);
        return;
    }
    // the row's key block, rotated by the row index: workgroups reach the XCDs round-robin by linear id, so
    // with gridDim.x a multiple of 8 block x of every row would land on XCD x % 8 and the partial last blocks
    // of ragged rows would pile onto the low XCDs; rotated, each row's blocks start on a different XCD
    const int64_t xb = ((int64_t)blockIdx.x + b) % gridDim.x;
    const int64_t key0 = xb * kKeysPerBlock;
    if (key0 >= n) return;

    // this wave's pages: logical pages lp0 .. lp0 + 3 of the row's sequence
    const int64_t lp0 = key0 / kPage + (int64_t)kPagesPerWave * wave;
    const int64_t tb = row_seq ? (int64_t)row_seq[b] : b;
    int64_t page[kPagesPerWave];
    bool page_ok[kPagesPerWave];
#pragma unroll
    for (int i = 0; i < kPagesPerWave; ++i) {
        const bool used = (lp0 + i) * kPage < n;
        const int32_t p = used ? block_table[tb * max_blocks + lp0 + i] : 0;
        page_ok[i] = p >= 0 && p < n_pages;
        if (used && !page_ok[i] && lane == 0) flag_error(err, SA_DEVERR_BLOCK_TABLE);
        page[i] = page_ok[i] ? p : 0;  // an unused or bad page is read from page 0 and ignored
    }

    // half-page h: keys 32 (h % 2) + l % 32 of page h / 2; lane l reads dims 16 ks + 8 (l / 32)
    auto load_half = [&](int h, bf16x8 (&bf)[kD / 16]) {
        const uint16_t *src = kidx_pages + (page[h / 2] * kPage + 32 * (h % 2) + lane % 32) * (int64_t)kD +
                              8 * (lane / 32);
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) bf[ks] = as_bf16x8(load16(src + 16 * ks));
    };
    bf16x8 bc[kD / 16], bn[kD / 16];
    load_half(0, bc);  // the first keys are in flight while q goes to LDS

    // q fragments: thread i moves fragments i, i + 256, i + 512, i + 768 (fragment f = (8 mt + ks) * 64 + l
    // holds q row 32 mt + l % 32, dims 16 ks + 8 (l / 32))
    const uint16_t *qr = q_idx + b * (int64_t)kH * kD;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int f = tid + u * kIdxThreads, l = f % kWave, mk = f / kWave;
        sh.qf[f] = load16(qr + (32 * (mk / 8) + l % 32) * kD + 16 * (mk % 8) + 8 * (l / 32));
    }
    if (tid < kH / 4) sh.wq[tid] = *reinterpret_cast<const float4 *>(w + b * kH + 4 * tid);
    for (int i = tid; i < kBins; i += kIdxThreads) sh.hist[i] = 0;
    __syncthreads();

#pragma unroll
    for (int h = 0; h < 2 * kPagesPerWave; ++h) {
        const int64_t kbase = (lp0 + h / 2) * kPage + 32 * (h % 2);
        if (h + 1 < 2 * kPagesPerWave) load_half(h + 1, bn);
        if (kbase < n) {  // uniform over the wave
            f32x16 acc0 = {}, acc1 = {};
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
                const bf16x8 a0 = as_bf16x8(sh.qf[ks * kWave + lane]);
                const bf16x8 a1 = as_bf16x8(sh.qf[(8 + ks) * kWave + lane]);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bc[ks], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bc[ks], acc1, 0, 0, 0);
            }
            // register g of lane l: head 32 mt + 8 (g / 4) + 4 (l / 32) + g % 4, key l % 32.  The terms are
            // summed in the fused prefill kernel's order (g ascending, the two head tiles alternating), so a
            // query row gets bit-identical scores from either kernel.
            float part = 0.f;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const float4 w0 = sh.wq[8 * gq / 4 + lane / 32];
                const float4 w1 = sh.wq[(32 + 8 * gq) / 4 + lane / 32];
                part = fmaf(w0.x, relu(acc0[4 * gq]), part);
                part = fmaf(w1.x, relu(acc1[4 * gq]), part);
                part = fmaf(w0.y, relu(acc0[4 * gq + 1]), part);
                part = fmaf(w1.y, relu(acc1[4 * gq + 1]), part);
                part = fmaf(w0.z, relu(acc0[4 * gq + 2]), part);
                part = fmaf(w1.z, relu(acc1[4 * gq + 2]), part);
                part = fmaf(w0.w, relu(acc0[4 * gq + 3]), part);
                part = fmaf(w1.w, relu(acc1[4 * gq + 3]), part);
            }
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                             false, false);
            float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if (!page_ok[h / 2]) score = -__builtin_inff();
            const int64_t s = kbase + lane;
            if (lane < 32 && s < n) {
                reinterpret_cast<float *>(sh.sc[wave])[32 * h + lane] = score;
                atomicAdd(&sh.hist[order_key(score) >> kBinShift], 1u);
            }
        }
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) bc[ks] = bn[ks];
    }
    // The scores leave in one 1 KB store per wave, after the loop: a store issued between the halves
    // would be waited for before the next half's MFMAs (loads and stores share one counter).  The store
    // is non-temporal: the scores are read once, by the next kernel.
    {
        const float4 v = sh.sc[wave][lane];  // the wave's own LDS rows: no barrier needed
        const int64_t s0 = lp0 * kPage + 4 * lane;
        float *dst = scores + b * ld + s0;
        if (s0 + 3 < n) {
            __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4 *>(dst));
        } else {
            if (s0 < n) dst[0] = v.x;
            if (s0 + 1 < n) dst[1] = v.y;
            if (s0 + 2 < n) dst[2] = v.z;
        }
        if (pmax_g) {
            // the largest score of each of the wave's pages as an order key (a page is the 16 lanes
            // of one DPP row; tokens past the context count as key 0, below every score's key)
            uint32_t x = s0 < n ? order_key(v.x) : 0u;
            x = max(x, s0 + 1 < n ? order_key(v.y) : 0u);
            x = max(x, s0 + 2 < n ? order_key(v.z) : 0u);
            x = max(x, s0 + 3 < n ? order_key(v.w) : 0u);
            x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true));  // row_shr:1
            x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true));  // row_shr:2
            x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true));  // row_shr:4
            x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true));  // row_shr:8
            const int64_t lp = lp0 + lane / 16;
            if ((lane & 15) == 15 && lp * kPage < n) pmax_g[b * pmax_ld + lp] = x;
        }
    }
    __syncthreads();
    for (int i = tid; i < kBins; i += kIdxThreads) {
        const uint32_t c = sh.hist[i];
        if (c) atomicAdd(&hist_g[b * kBins + i], c);
    }
}

// Where the chunks of one sequence meet: the sequence's candidate list ([B, kCap] keys and indices), each
// chunk's (offset, count) in it, and per sequence the list's fill and the number of chunks done.
struct TopkMeet {
    uint32_t *keys;
    int32_t *idx;
    int32_t *info;  // [B, n_chunks, 2]
    uint32_t *sync;  // [B, 2], zero at launch
    int64_t n_chunks;
};

// Workgroup (c, b): tokens [32768 c, 32768 (c + 1)) of sequence b.  The threshold bin b* from the sequence's
// histogram, then every score of the chunk in bins >= b* appended to an LDS list in token order.  The scores
// stream in rounds of 16384 (4 coalesced float4 loads per thread, the chunk's second round in flight while
// the first is compacted); one barrier per round orders the candidates: sub-round u of a round covers 4096
// consecutive tokens in thread order, and the per-(sub-round, wave) counts published in LDS give each wave
// its offset.  A sequence of one chunk selects from its LDS list at once.  Otherwise each chunk reserves a
// stretch of the sequence's global list (atomic add on its fill) and copies its candidates there; the last
// chunk to arrive (its arrival count is a release / acquire at device scope, which the XCDs' separate L2s
// need) gathers the stretches in chunk order, so the list is in token order as one workgroup would have
// built it, and selects.  A sequence whose candidates exceed kCap is selected from its full score row by
// its first chunk alone.
__global__ __launch_bounds__(kTopkThreads) void decode_topk_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ ctx_len, int32_t max_ctx,
    const int32_t *__restrict__ topk_b, int32_t max_topk, const uint32_t *__restrict__ hist_g, TopkMeet meet,
    int32_t *__restrict__ idx, uint32_t *err)
{
    __shared__ uint32_t ck[kCap];
    __shared__ int32_t ci[kCap];
    __shared__ topk::SelectShared<kTopkWaves> sh;
    __shared__ int counts[2][kSubRounds][kTopkWaves];
    __shared__ int info[3];
    __shared__ int meet_sh[2];
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int64_t b = blockIdx.y;
    const int c = blockIdx.x;
    int32_t *dst = idx + b * max_topk;
    int64_t n, m;
    if (!decode_row_ok(ctx_len, topk_b, max_ctx, max_topk, b, &n, &m)) {
        if (c == 0) {
            if (tid == 0) flag_error(err, SA_DEVERR_TOPK);
            for (int i = tid; i < max_topk; i += kTopkThreads) dst[i] = -1;
        }
        return;
    }
    if (m == n) {  // every visible token is selected
        if (c == 0)
            for (int i = tid; i < max_topk; i += kTopkThreads) dst[i] = i < n ? i : -1;
        return;
    }
    const int32_t n32 = (int32_t)n;  // n <= max_ctx < 2^31
    const int n_chunks = (n32 + kTopkChunk - 1) / kTopkChunk;
    if (c >= n_chunks) return;
    const float *row = scores + b * ld;
    const int32_t c0 = c * kTopkChunk, c1 = c0 + kTopkChunk < n32 ? c0 + kTopkChunk : n32;

    // Sub-round u of the round at `base`: thread t holds tokens base + 4096 u + 4 t .. +3.  Every load is
    // issued, also past the chunk's end (it then reads the chunk's first 16 bytes, never used).
    float4 v0[kSubRounds], v1[kSubRounds];
    auto load_round = [&](float4 (&v)[kSubRounds], int32_t base) {
#pragma unroll
        for (int u = 0; u < kSubRounds; ++u) {
            const int32_t p = base + u * 4 * kTopkThreads + 4 * tid;
            v[u] = *reinterpret_cast<const float4 *>(row + (p < c1 ? p : c0));
        }
    };
    load_round(v0, c0);  // in flight while wave 0 finds the threshold bin
    load_round(v1, c0 + kRoundScores);
    if (tid < kWave) {
        int above, upto;
        const int bin = topk::threshold_bin(hist_g + b * kBins, (int)m, &above, &upto);
        if (tid == 0) {
            info[0] = bin;
            info[1] = above;
            info[2] = upto;
        }
    }
    __syncthreads();
    const int bin = info[0], above = info[1], upto = info[2];
    if (upto > kCap) {
        if (c == 0) {
            topk::select_and_emit(sh, topk::GlobalScores{row}, (int)n, bin, above, (int)m, dst);
            for (int i = (int)m + tid; i < max_topk; i += kTopkThreads) dst[i] = -1;
        }
        return;
    }

    // order_key(f) >= key_lo as one unsigned compare on the raw bits u of f: (u ^ X) >= Y.  Above
    // the +0.0 bin it is a signed compare of u with key_lo's magnitude; at or below it, u <= C (the
    // +0.0 bin also takes -0.0, which order_key maps to +0.0).
    const uint32_t key_lo = (uint32_t)bin << kBinShift;
    uint32_t X, Y;
    if (key_lo > 0x80000000u) {
        X = 0x80000000u;
        Y = (key_lo & 0x7FFFFFFFu) ^ 0x80000000u;
    } else {
        const uint32_t C = key_lo == 0x80000000u ? 0x80000000u : ~key_lo;
        X = 0xFFFFFFFFu;
        Y = ~C;
    }
    int total = 0;  // candidates appended so far
    int rnd = 0;    // rounds done (the parity picks the counts buffer)
    // append the candidates of the round at `base` (held in v)
    auto compact_round = [&](const float4 (&v)[kSubRounds], int32_t base) {
        const int par = rnd & 1;
        const bool tail = base + kRoundScores > c1;  // uniform: only then may tokens lie past the chunk
        uint32_t selm = 0;  // bit 4 u + i: token base + 4096 u + 4 tid + i is a candidate
#pragma unroll
        for (int u = 0; u < kSubRounds; ++u) {
            const int32_t p = base + u * 4 * kTopkThreads + 4 * tid;
            const uint32_t w[4] = {__float_as_uint(v[u].x), __float_as_uint(v[u].y), __float_as_uint(v[u].z),
                                   __float_as_uint(v[u].w)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bool pass = (w[i] ^ X) >= Y;
                if (tail) pass = pass && p + i < c1;
                selm |= (pass ? 1u : 0u) << (4 * u + i);
            }
        }
        int pre[kSubRounds];  // candidates of sub-round u in this wave's lower lanes
#pragma unroll
        for (int u = 0; u < kSubRounds; ++u) {
            const int cnt = __popc((selm >> (4 * u)) & 0xFu);
            const int incl = topk::wave_incl_scan(cnt);
            pre[u] = incl - cnt;
            if (lane == kWave - 1) counts[par][u][wave] = incl;
        }
        __syncthreads();
        // Offsets in (sub-round, wave) order: lane l of every wave takes the count of sub-round l / 16,
        // wave l % 16, and one scan over the wave gives all 64 offsets.
        const int cl = counts[par][lane / kTopkWaves][lane % kTopkWaves];
        const int cincl = topk::wave_incl_scan(cl);
        const int cexcl = cincl - cl;
#pragma unroll
        for (int u = 0; u < kSubRounds; ++u) {
            int pos = total + __builtin_amdgcn_readlane(cexcl, kTopkWaves * u + wave) + pre[u];
            const int32_t p = base + u * 4 * kTopkThreads + 4 * tid;
            const uint32_t w0 = __float_as_uint(v[u].x), w1 = __float_as_uint(v[u].y);
            const uint32_t w2 = __float_as_uint(v[u].z), w3 = __float_as_uint(v[u].w);
            for (uint32_t bits = (selm >> (4 * u)) & 0xFu; bits; bits &= bits - 1) {
                const int i = __builtin_ctz(bits);
                // element i picked with masks, not a select (which the compiler may turn into an
                // indexed access that forces the buffer out of registers)
                const uint32_t f = (w0 & (0u - (i == 0))) | (w1 & (0u - (i == 1))) | (w2 & (0u - (i == 2))) |
                                   (w3 & (0u - (i == 3)));
                if (pos < kCap) {
                    ck[pos] = order_key(__uint_as_float(f));
                    ci[pos] = p + i;
                }
                ++pos;
            }
        }
        total += __builtin_amdgcn_readlane(cincl, kWave - 1);
        ++rnd;
    };
    compact_round(v0, c0);
    if (c0 + kRoundScores < c1) compact_round(v1, c0 + kRoundScores);
    __syncthreads();
    if (total > kCap) total = kCap;  // not reached: the chunks' candidates add up to at most upto <= kCap

    if (n_chunks > 1) {
        uint32_t *fill = meet.sync + 2 * b, *arrived = fill + 1;
        int32_t *cinfo = meet.info + 2 * (b * meet.n_chunks);
        uint32_t *gk = meet.keys + b * kCap;
        int32_t *gi = meet.idx + b * kCap;
        if (tid == 0) {
            const int off = (int)atomicAdd(fill, (uint32_t)total);
            cinfo[2 * c] = off;
            cinfo[2 * c + 1] = total;
            meet_sh[0] = off;
        }
        __syncthreads();
        const int off = meet_sh[0];
        for (int i = tid; i < total && off + i < kCap; i += kTopkThreads) {
            gk[off + i] = ck[i];
            gi[off + i] = ci[i];
        }
        // The barrier orders every wave's stores before thread 0's arrival; the arrival is a release (this
        // workgroup's list and info, device-wide) and an acquire (every earlier chunk's), made once for the
        // workgroup: the cache write-back and invalidation it implies are cache-wide, not per wave.
        __syncthreads();
        if (tid == 0) {
            const uint32_t before =
                __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            meet_sh[1] = before == (uint32_t)(n_chunks - 1);
        }
        __syncthreads();
        if (!meet_sh[1]) return;
        total = 0;
        for (int cc = 0; cc < n_chunks; ++cc) {
            const int o = cinfo[2 * cc], k = cinfo[2 * cc + 1];
            for (int i = tid; i < k && total + i < kCap && o + i < kCap; i += kTopkThreads) {
                ck[total + i] = gk[o + i];
                ci[total + i] = gi[o + i];
            }
            total += k;
        }
        if (total > kCap) total = kCap;
        if (tid == 0) {  // ready for the next call (the reset kernel clears them too)
            *fill = 0;
            *arrived = 0;
        }
        __syncthreads();
    }
    topk::select_and_emit_inline(sh, topk::LdsCands{ck, ci}, total, bin, above, (int)m, dst);
    for (int i = (int)m + tid; i < max_topk; i += kTopkThreads) dst[i] = -1;
}

}  // namespace

DecodeTopkLayout decode_topk_layout(int64_t B, int64_t max_ctx)
{
    DecodeTopkLayout l;
    l.ld = (max_ctx + 63) / 64 * 64;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t off = at;
        at += (bytes + 255) / 256 * 256;
        return off;
    };
    l.scores = take((size_t)B * l.ld * sizeof(float));
    l.hist = take((size_t)B * kBins * sizeof(uint32_t));
    l.pmax_ld = l.ld / kPage;
    l.pmax = take((size_t)B * l.pmax_ld * sizeof(uint32_t));
    l.n_chunks = (max_ctx + kTopkChunk - 1) / kTopkChunk;
    l.cand_keys = take((size_t)B * kCap * sizeof(uint32_t));
    l.cand_idx = take((size_t)B * kCap * sizeof(int32_t));
    l.chunk_info = take((size_t)B * l.n_chunks * 2 * sizeof(int32_t));
    l.sync = take((size_t)B * 2 * sizeof(uint32_t));
    l.total = at;
    return l;
}

hipError_t launch_decode_indexer(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                                 int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                 const int32_t *ctx_len, const int32_t *row_seq, int32_t B, int32_t max_ctx,
                                 bool page_maxima, void *ws, hipStream_t st)
{
    const DecodeTopkLayout l = decode_topk_layout(B, max_ctx);
    char *base = reinterpret_cast<char *>(ws);
    float *scores = reinterpret_cast<float *>(base + l.scores);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base + l.hist);
    uint32_t *pmax = page_maxima ? reinterpret_cast<uint32_t *>(base + l.pmax) : nullptr;
    {
        const int64_t nz = (int64_t)B * kBins;
        hipLaunchKernelGGL(decode_reset_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, hist,
                           reinterpret_cast<uint32_t *>(base + l.sync), (int64_t)B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        KernelTimer timer(h, SA_KERNEL_INDEXER, st);
        dim3 grid((unsigned)((max_ctx + kKeysPerBlock - 1) / kKeysPerBlock), (unsigned)B);
        hipLaunchKernelGGL(indexer_decode_kernel, grid, dim3(kIdxThreads), 0, st,
                           reinterpret_cast<const uint16_t *>(q_idx), w,
                           reinterpret_cast<const uint16_t *>(kidx_pages), n_pages, block_table, max_blocks,
                           ctx_len, row_seq, max_ctx, scores, l.ld, hist, pmax, l.pmax_ld, h.d_err);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_decode_indexer_topk(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                      const int32_t *ctx_len, const int32_t *topk_b, int32_t B, int32_t max_ctx,
                                      int32_t *idx, void *ws, hipStream_t st)
{
    hipError_t e = launch_decode_indexer(h, q_idx, w, kidx_pages, n_pages, block_table, max_blocks, ctx_len,
                                         nullptr, B, max_ctx, false, ws, st);
    if (e != hipSuccess) return e;
    return launch_decode_topk(h, ctx_len, topk_b, h.cfg.max_topk, B, max_ctx, idx, ws, st);
}

hipError_t launch_decode_topk(sa_handle_s &h, const int32_t *ctx_len, const int32_t *topk_b, int32_t max_topk,
                              int32_t B, int32_t max_ctx, int32_t *idx, void *ws, hipStream_t st)
{
    const DecodeTopkLayout l = decode_topk_layout(B, max_ctx);
    char *base = reinterpret_cast<char *>(ws);
    const float *scores = reinterpret_cast<const float *>(base + l.scores);
    const uint32_t *hist = reinterpret_cast<const uint32_t *>(base + l.hist);
    const TopkMeet meet{reinterpret_cast<uint32_t *>(base + l.cand_keys), reinterpret_cast<int32_t *>(base + l.cand_idx),
                        reinterpret_cast<int32_t *>(base + l.chunk_info), reinterpret_cast<uint32_t *>(base + l.sync),
                        l.n_chunks};
    KernelTimer timer(h, SA_KERNEL_TOPK, st);
    hipLaunchKernelGGL(decode_topk_kernel, dim3((unsigned)l.n_chunks, (unsigned)B), dim3(kTopkThreads), 0, st,
                       scores, l.ld, ctx_len, max_ctx, topk_b, max_topk, hist, meet, idx, h.d_err);
    return hipGetLastError();
}

}  // namespace sa
