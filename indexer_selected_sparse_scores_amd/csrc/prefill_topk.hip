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
//  * Keys stream through LDS in 64-key tiles (16 KB, three buffers) stored in MFMA fragment
//    order, so that a B fragment is one linear, conflict-free 16-byte read per lane.  Per
//    tile each wave issues 32 v_mfma_f32_32x32x16_bf16: heads on M (2 tiles of 32), keys on
//    N (2 tiles of 32), d_I on K, fp32 accumulation.  B fragments flow through a 4-deep
//    register ring read 3 k-steps ahead; the third buffer lets the ring run into the next
//    tile before the tile barrier.
//  * Epilogue in registers: each lane holds 16 head rows of one key column per 32x32 tile;
//    ReLU, the weight and the head sum run in-lane, one v_permlane32_swap finishes the head
//    sum and leaves lane l with the score of key tile_base + l.
//  * Streaming top-k: a per-row 2048-bin LDS histogram of the order-preserving keys' top 11
//    bits gives the wave a running threshold bin: once m scores lie in bins >= b, no score in a
//    lower bin can be selected.  Only scores in bins >= the running threshold are counted and
//    appended (ballot-compacted, in key order) to the row's candidate list in the workspace --
//    about m (1 + ln(t/m)) of the t+1 scores.
//  * Query rows may be a chunk of a longer sequence (positions pos0 ..), and the keys may come from
//    the 64-token pages of the sequence's block-table row: a key tile is then one page, whose pool
//    page is looked up once per row tile and kept in LDS (chunked prefill against a paged cache).
//  * At the end of the tile the final histogram fixes the threshold bin b* exactly.  The
//    candidates in bins >= b* are gathered into LDS (at most kCap; otherwise the list is
//    scanned in global memory), an MSD radix select over the remaining 21 key bits finds the
//    exact m-th key, and an ordered compaction writes the selection in ascending key order.
#include <type_traits>

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
constexpr int kSteps = kHalves * (kD / 16);  // k-steps (B fragments) per tile (16)
constexpr int kRing = 4;            // B fragments in flight per wave
constexpr int kBufs = 3;            // LDS key tiles
constexpr int kTileLoads = kKT * 16 / 512;  // 16-byte chunks each thread moves per tile
constexpr int kChunks = kD * 2 / 16;  // 16-byte chunks per key row (16)
constexpr int kRefresh = 32;        // key tiles between running-threshold refreshes
static_assert(kSteps % kRing == 0, "ring slots repeat every tile");
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt not waited on
using topk::kBins;
using topk::kBinShift;
using topk::kCap;
using topk::kPerThread;

static_assert(kRows * kBins * 4 == kCap * 8, "the histogram region holds the candidates");

template <bool kPaged>
struct Shared {
    uint4 keys[kBufs][kKT * kChunks];    // key tiles in fragment order
    uint32_t region[kRows * kBins];      // 64 KB: histograms, then candidate (key, index)
    topk::SelectShared<kRows> sel;
    int info[kRows][4];                  // per row: b*, count in bins > b*, count in bins >= b*,
                                         // candidate list length
    int tile;
    int32_t pages[kPaged ? kPrefillMaxPages : 1];  // pool page of each 64-key tile (-1: bad entry)
};

// One row tile of a batch of sequences (32 bytes): rows q0 .. min(q0 + 8, len) - 1 of sequence seq.
struct VarlenTile {
    int32_t seq, q0, len, pos0, rowbase, pad[3];
};

// One row tile of query rows that name their own (sequence, position): n <= 8 rows of sequence seq, with
// their row indices in q_idx, w and idx and their positions, in ascending position order (72 bytes).
struct RowTile {
    int32_t seq, n;
    int32_t row[kRows], pos[kRows];
};

// Where the index keys come from: contiguous rows, or the 64-token pages of one sequence's block-table
// row (a key tile is exactly one page).  With a tile table (a batch of sequences) or a row table (rows
// naming their own sequence and position), each row tile names its sequence, whose block-table row is
// table + seq * table_ld.
struct KeySource {
    const uint16_t *base;
    const int32_t *table;   // paged: the sequence's block-table row (tile / row table: the whole block table)
    int64_t n_pages;
    uint32_t *err;
    const VarlenTile *tiles = nullptr;
    int64_t table_ld = 0;
    const RowTile *rows = nullptr;
};

// Key tile layout: the 16-byte piece holding dims 8 j .. 8 j + 7 of key r sits at
// ((r / 32) * 8 + j / 2) * 64 + (j % 2) * 32 + r % 32, so that the B fragment of k-step i of a
// tile (keys 32 (i / 8) + l % 32, dims 16 (i % 8) + 8 (l / 32)) is piece 64 i + l of lane l.
__device__ __forceinline__ int piece_slot(int r, int j)
{
    return ((r >> 5) * 8 + (j >> 1)) * 64 + (j & 1) * 32 + (r & 31);
}

// Chunk c of a tile load (c = thread + 512 u): 16 consecutive lanes take 16 consecutive keys
// at one 16-byte column, so the fragment-order LDS store of a wave is conflict-free.
__device__ __forceinline__ int chunk_key(int c) { return (c & 15) + 16 * ((c >> 6) & 3); }
__device__ __forceinline__ int chunk_col(int c) { return ((c >> 4) & 3) + 4 * (c >> 8); }

// Scheduling pattern of one k-step: two MFMAs with 4 epilogue VALU ops after each, and the
// ring read of a later k-step after the MFMAs that free its slot.
__device__ __forceinline__ void step_pattern()
{
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
}

// Selection of one row from its candidate list (nl entries of (order key, index) in index order, every
// score in bins >= `bin` among them, upto <= kCap of those) by the whole workgroup, with the LDS of the
// key tiles as scratch (the tiles are not in use between row tiles):
//  * gather: the list streams in rounds of 4096 entries (entry base + 512 u + thread, u = 0..7: every
//    load instruction reads 512 contiguous bytes), two rounds in flight; the entries in bins >= bin go
//    to LDS in index order -- per round, the per-(u, wave) counts published in LDS give every wave its
//    offsets with one scan over 64 lanes -- and those in bin `bin` itself count their next 11 key bits
//    (bits 20..10) in a 2048-bin histogram;
//  * from it one wave finds the 11-bit digit holding the (m - above)-th largest key of the bin, a
//    second pass over the gathered keys counts the last 10 bits of those with that digit, and one wave
//    finds the exact key tau of the m-th largest score;
//  * ordered emit: every key > tau and the first `need` keys == tau in index order, in rounds of 4096
//    gathered entries with the same (u, wave) offsets.
struct RowSelScratch {
    uint32_t hist[kBins];
    int counts[2][8][kRows];  // per round parity: entries kept per (u, wave)
    int eq[2][8][kRows];      // emit: keys == tau per (u, wave)
    int digit, need;
};

typedef __attribute__((address_space(3))) RowSelScratch lds_sel_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(1))) const uint64_t glb_cu64;  // a (key, index) pair, key in the low word
typedef __attribute__((address_space(1))) int32_t glb_i32;

// Out of line, with LDS and global pointers named as such: the fused kernel's tile loop keeps its whole
// register budget (inlined, this code made the allocator spill a pointer the loop reloads), and the
// accesses stay LDS and global instructions.
__device__ __noinline__ void select_row_lds(lds_sel_t *ss, lds_u32 *ck, lds_i32 *ci, glb_cu64 *list, int nl,
                                            int bin, int above, int m, glb_i32 *dst)
{
    static_assert(kRows * 8 == kWave, "one lane per (u, wave) count");
    constexpr int kU = 8;                    // entries per thread per round
    constexpr int kRound = kU * kThreads;    // 4096
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const uint32_t lo = (uint32_t)bin << kBinShift;
    auto lds_inc = [](lds_u32 *p) { __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); };
    // offsets of (u, wave) from the counts of one round: exclusive scan in (u, wave) order
    auto offsets = [&](const __attribute__((address_space(3))) int (*cnt)[kRows], int &excl, int &total) {
        const int cl = cnt[lane >> 3][lane & 7];
        const int incl = topk::wave_incl_scan(cl);
        excl = incl - cl;
        total = __builtin_amdgcn_readlane(incl, kWave - 1);
    };

    for (int i = tid; i < kBins; i += kThreads) ss->hist[i] = 0;
    __syncthreads();
    uint2 v0[kU], v1[kU];
    auto load_round = [&](uint2 (&v)[kU], int base) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int j = base + u * kThreads + tid;
            const uint64_t e = list[j < nl ? j : 0];
            v[u] = make_uint2((uint32_t)e, (uint32_t)(e >> 32));
        }
    };
    int out = 0, rnd = 0;
    auto gather_round = [&](const uint2 (&v)[kU], int base) {
        const int par = rnd & 1;
        uint32_t selm = 0;
        int pre[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const bool keep = base + u * kThreads + tid < nl && v[u].x >= lo;
            if (keep && (v[u].x >> kBinShift) == (uint32_t)bin) lds_inc(&ss->hist[(v[u].x >> 10) & (kBins - 1)]);
            const uint64_t b = __ballot(keep);
            pre[u] = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            if (lane == 0) ss->counts[par][u][wave] = __popcll(b);
            selm |= (keep ? 1u : 0u) << u;
        }
        __syncthreads();
        int excl, total;
        offsets(ss->counts[par], excl, total);
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if ((selm >> u) & 1u) {
                const int pos = out + __builtin_amdgcn_readlane(excl, 8 * u + wave) + pre[u];
                if (pos < kCap) {
                    ck[pos] = v[u].x;
                    ci[pos] = (int32_t)v[u].y;
                }
            }
        out += total;
        ++rnd;
    };
    load_round(v0, 0);
    if (nl > kRound) load_round(v1, kRound);
#pragma unroll 1
    for (int base = 0; base < nl; base += 2 * kRound) {
        gather_round(v0, base);
        if (base + 2 * kRound < nl) load_round(v0, base + 2 * kRound);
        if (base + kRound >= nl) break;
        gather_round(v1, base + kRound);
        if (base + 3 * kRound < nl) load_round(v1, base + 3 * kRound);
    }
    const int n = out < kCap ? out : kCap;  // == upto

    // bits 20..10 of the m-th key (the histogram is complete: every atomic precedes a round's barrier)
    const int need0 = m - above;  // >= 1 keys of bin `bin` to take
    if (tid < kWave) {
        int ab;
        const int d = topk::threshold_bin((const uint32_t *)ss->hist, need0, &ab, nullptr);
        if (tid == 0) {
            ss->digit = d;
            ss->need = need0 - ab;
        }
    }
    __syncthreads();
    const uint32_t d1 = (uint32_t)ss->digit;
    const int need1 = ss->need;
    __syncthreads();  // every wave has read the digit before the histogram is cleared
    for (int i = tid; i < kBins; i += kThreads) ss->hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = ((uint32_t)bin << 11) | d1;  // key >> 10 of the keys still in play
    for (int j = tid; j < n; j += kThreads) {
        const uint32_t key = ck[j];
        if ((key >> 10) == prefix) lds_inc(&ss->hist[key & 1023u]);
    }
    __syncthreads();
    if (tid < kWave) {
        int ab;
        const int d = topk::threshold_bin((const uint32_t *)ss->hist, need1, &ab, nullptr);
        if (tid == 0) {
            ss->digit = d;
            ss->need = need1 - ab;
        }
    }
    __syncthreads();
    const uint32_t tau = (prefix << 10) | (uint32_t)ss->digit;  // exact key of the m-th largest score
    const int need = ss->need;                                    // keys == tau to take, lowest indices first

    // ordered emit
    int eq_before = 0, taken = 0;
    rnd = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += kRound) {
        const int par = rnd & 1;
        uint32_t gtm = 0, eqm = 0;
        int eq_pre[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int j = base + u * kThreads + tid;
            const bool in = j < n;
            const uint32_t key = in ? ck[j] : 0u;
            const bool gt = in && key > tau, eq = in && key == tau;
            const uint64_t b = __ballot(eq);
            eq_pre[u] = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            if (lane == 0) ss->eq[par][u][wave] = __popcll(b);
            gtm |= (gt ? 1u : 0u) << u;
            eqm |= (eq ? 1u : 0u) << u;
        }
        __syncthreads();
        int eq_excl, eq_total;
        offsets(ss->eq[par], eq_excl, eq_total);
        uint32_t take = gtm;
        int pre[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int rank = eq_before + __builtin_amdgcn_readlane(eq_excl, 8 * u + wave) + eq_pre[u];
            if (((eqm >> u) & 1u) && rank < need) take |= 1u << u;
            const uint64_t b = __ballot((take >> u) & 1u);
            pre[u] = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            if (lane == 0) ss->counts[par][u][wave] = __popcll(b);
        }
        __syncthreads();
        int t_excl, t_total;
        offsets(ss->counts[par], t_excl, t_total);
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if ((take >> u) & 1u) {
                const int pos = taken + __builtin_amdgcn_readlane(t_excl, 8 * u + wave) + pre[u];
                if (pos < m) dst[pos] = ci[base + u * kThreads + tid];
            }
        eq_before += eq_total;
        taken += t_total;
        ++rnd;
    }
}

// Block keys instead of a selection (the first pass of the two-tier selection): for every row that has
// more than `need` visible keys, the order key of the best visible score of each 64-key tile it sees.
struct BlockKeysOut {
    uint32_t *keys;    // [L, ld]: row i, tile j
    int64_t ld;
};

// Query rows i = 0 .. L-1 are the tokens at positions pos0 + i of one sequence; keys are its tokens
// 0 .. pos0 + L - 1 (contiguous rows, or pages of its block-table row when kPaged).  Rows with at most
// `need` visible keys are not scored (need = topk: all their keys are selected).
// With a tile table (kPaged only), tile e = ks.tiles[e] holds rows q0 .. q0 + 7 (< len) of sequence seq,
// whose len query rows sit at rows rowbase .. of q_idx, w and idx and at positions pos0 .. pos0 + len - 1.
template <bool kPaged, bool kBlockKeys>
__global__ __launch_bounds__(kThreads, 1) void indexer_topk_prefill_kernel(
    const uint16_t *__restrict__ q_idx_all, const float *__restrict__ w_all, KeySource ks, int64_t L_all,
    int64_t pos0_all, int32_t topk, int64_t need, int32_t *__restrict__ idx_all, uint2 *__restrict__ cands,
    int64_t cand_ld, BlockKeysOut bk, int32_t *__restrict__ counter, int32_t n_tiles)
{
    __shared__ Shared<kPaged> sh;
    const uint16_t *__restrict__ k_idx = ks.base;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    uint2 *my_cands = cands + ((int64_t)blockIdx.x * kRows + wave) * cand_ld;

#pragma unroll 1
    for (;;) {
        if (tid == 0) sh.tile = atomicAdd(counter, 1);
        __syncthreads();
        const int it = __builtin_amdgcn_readfirstlane(sh.tile);
        if (it >= n_tiles) break;
        int64_t q0 = (int64_t)(n_tiles - 1 - it) * kRows;  // latest rows first
        int64_t L = L_all, pos0 = pos0_all, rb = 0;         // this tile's sequence, and its first query row
        const int32_t *table = ks.table;
        const RowTile *rt = nullptr;  // row table: each row's own query row and position
        if constexpr (kPaged) {
            if (ks.tiles) {
                const VarlenTile vt = ks.tiles[n_tiles - 1 - it];
                if (vt.len <= 0) {  // unused entry; the barrier keeps sh.tile until every thread has read it
                    __syncthreads();
                    continue;
                }
                q0 = vt.q0;
                L = vt.len;
                pos0 = vt.pos0;
                rb = vt.rowbase;
                table = ks.table + (int64_t)vt.seq * ks.table_ld;
            } else if (ks.rows) {
                rt = ks.rows + (n_tiles - 1 - it);
                const int32_t nr = rt->n;
                if (nr <= 0) {  // unused entry
                    __syncthreads();
                    continue;
                }
                q0 = 0;
                L = nr;
                table = ks.table + (int64_t)rt->seq * ks.table_ld;
            }
        }
        // query row (index into q_idx_all, w_all, idx_all) and position of row r < L - q0 of the tile
        auto abs_row = [&](int r) -> int64_t { return rt ? (int64_t)rt->row[r] : rb + q0 + r; };
        auto pos_of = [&](int r) -> int64_t { return rt ? (int64_t)rt->pos[r] : pos0 + q0 + r; };
        const int n_rows = (int)(L - q0 < kRows ? L - q0 : kRows);
        // position of the tile's last row (keys 0 .. t_last are streamed; positions ascend within a tile)
        const int64_t t_last = pos_of(n_rows - 1);
        const int64_t ri = q0 + wave;    // this wave's query row within the call (block keys) or tile
        const bool row_ok = wave < n_rows;
        const int64_t row = row_ok ? pos_of(wave) : 0;   // its position: it sees keys 0 .. row
        const int m = row_ok ? (int)((int64_t)topk < row + 1 ? (int64_t)topk : row + 1) : 0;
        const bool selects = row_ok && row + 1 > need;  // fewer than all visible keys
        int n_cand = 0;                                   // this row's candidate list length

        if (t_last + 1 > need) {  // some row of the tile needs scores
            if constexpr (!kBlockKeys)
                for (int i = tid; i < kRows * kBins; i += kThreads) sh.region[i] = 0;
            if constexpr (kPaged) {
                // the pool page of every key tile of the prefix, checked once (a bad entry is read as page 0
                // and its keys score -inf)
                for (int j = tid; j <= (int)(t_last / kKT); j += kThreads) {
                    const int32_t pg = table[j];
                    const bool ok = pg >= 0 && pg < ks.n_pages;
                    if (!ok) flag_error(ks.err, SA_DEVERR_BLOCK_TABLE);
                    sh.pages[j] = ok ? pg : -1;
                }
                __syncthreads();
            }

            // A operand and weights of this wave's query row
            bf16x8 a[2][kD / 16];
            float wv[2][16];
            const int64_t qrow = abs_row(row_ok ? wave : n_rows - 1);
            const uint16_t *qr = q_idx_all + qrow * (int64_t)kH * kD;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int ks = 0; ks < kD / 16; ++ks)
                    a[mt][ks] = as_bf16x8(load16(qr + (32 * mt + lane % 32) * kD + 16 * ks + 8 * (lane / 32)));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int g = 0; g < 16; ++g)
                    wv[mt][g] = w_all[qrow * kH + 32 * mt + 8 * (g / 4) + 4 * (lane / 32) + g % 4];

            // key tile loader: thread i moves chunks i and i + 512 of the 1024 in a tile
            const int n_kt = (int)(t_last / kKT) + 1;
            auto load_tile = [&](int kt, uint4 (&v)[kTileLoads]) {
                // paged: every key of tile kt (a clamped one too: t_last lies in the last tile) is in
                // page pages[kt], one uniform value per tile
                int64_t shift = 0;
                if constexpr (kPaged) {
                    const int32_t pg = __builtin_amdgcn_readfirstlane(sh.pages[kt]);
                    shift = ((int64_t)(pg >= 0 ? pg : 0) - kt) * kKT;
                }
                // uniform tile base and 32-bit lane offsets (keys past t_last read key t_last), so the
                // addressing stays in scalar registers but for one min and one shift-add per load
                const int64_t k0 = (int64_t)kt * kKT;
                const unsigned char *tbase = reinterpret_cast<const unsigned char *>(k_idx + (k0 + shift) * kD);
                const int lim = (int)(t_last - k0 < kKT ? t_last - k0 : kKT);
#pragma unroll
                for (int u = 0; u < kTileLoads; ++u) {
                    const int c = tid + u * kThreads;
                    const int key = chunk_key(c) < lim ? chunk_key(c) : lim;
                    v[u] = load16(tbase + (uint32_t)(key * (kD * 2) + 16 * chunk_col(c)));
                }
            };
            auto store_tile = [&](int buf, const uint4 (&v)[kTileLoads]) {
#pragma unroll
                for (int u = 0; u < kTileLoads; ++u) {
                    const int c = tid + u * kThreads;
                    sh.keys[buf][piece_slot(chunk_key(c), chunk_col(c))] = v[u];
                }
            };
            {
                uint4 v[kTileLoads];
                load_tile(0, v);
                store_tile(0, v);
                if (n_kt > 1) {
                    load_tile(1, v);
                    store_tile(1, v);
                }
            }
            uint32_t *hist = sh.region + wave * kBins;
            int run_bin = 0;  // running threshold bin: scores in lower bins are dropped
            // the score at the lower edge of run_bin (NaN for bin 0: every score is kept), so that the
            // window's test is one float compare, !(score < run_thr) <=> order_key(score) >> kBinShift >=
            // run_bin for every non-NaN score; a NaN score is kept whatever the bin (harmless: only bins at or
            // above the final threshold, never below run_bin, are read again)
            float run_thr = __builtin_nanf("");

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
            // the window's keys are s = sb - 32 (sb >= 0; 32-bit is enough: row < 2^31)
            const uint32_t vis_hi = (uint32_t)row + 32u;
            float prev_hi = -__builtin_inff();  // block keys: best score of the first half of the last tile
            auto finish_window = [&](float part_odd, float part_even, uint32_t sb) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part_odd),
                                                                 __float_as_uint(part_even), false, false);
                float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                const bool vis = sb >= 32u && sb <= vis_hi;
                const uint32_t s = sb - 32u;
                if constexpr (kPaged) {
                    // lanes 0-31 hold keys of tile kw - 1, lanes 32-63 of tile kw; keys of a bad page score -inf
                    const int kw = __builtin_amdgcn_readfirstlane((int)(sb / kKT));
                    const bool bad_lo = kw >= 1 && sh.pages[kw - 1] < 0;
                    const bool bad_hi = sh.pages[kw < kPrefillMaxPages ? kw : kPrefillMaxPages - 1] < 0;
                    if (vis && (lane < 32 ? bad_lo : bad_hi)) score = -__builtin_inff();
                }
                if constexpr (kBlockKeys) {
                    // lanes 0-31 finish tile kw - 1 (its first half was the previous window's lanes 32-63)
                    const int kw = __builtin_amdgcn_readfirstlane((int)(sb / kKT));
                    const float hm = half_wave_max(vis ? score : -__builtin_inff());
                    const float m_lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hm), 0));
                    const float m_hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hm), 32));
                    if (kw >= 1 && (int64_t)(kw - 1) * kKT <= row && lane == 0)
                        bk.keys[ri * bk.ld + kw - 1] = order_key(fmaxf(prev_hi, m_lo));
                    prev_hi = m_hi;
                    return;
                }
                // Only scores in bins >= the running threshold are counted and kept: the final threshold bin
                // is never below it (the threshold only rises, each time to a bin that at least m counted
                // scores reach), so the counts of every bin at or above the final one stay exact.  Late in a
                // long row most windows keep nothing and skip the LDS atomic altogether.
                const bool keep = vis && !(score < run_thr);
                const uint64_t ballot = __builtin_amdgcn_ballot_w64(keep);
                if (ballot) {
                    if (keep) {
                        const uint32_t key = order_key(score);
                        atomicAdd(&hist[key >> kBinShift], 1u);
                        const int rank = (int)__builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(ballot >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
                        my_cands[n_cand + rank] = make_uint2(key, s);
                    }
                    n_cand += __popcll(ballot);
                }
            };

            // B fragment ring: slot i % kRing holds k-step i of the tile being multiplied
            bf16x8 ring[kRing];
            // q and the weights have arrived: no wait on them is left inside the loop, where it
            // would also wait for the key loads in flight
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();  // tiles 0 and 1 stored
#pragma unroll
            for (int i = 0; i < kRing; ++i) ring[i] = as_bf16x8(sh.keys[0][64 * i + lane]);

            // One barrier per tile, between its two halves: by then every wave has finished tile
            // kt - 1 (so the buffer of tile kt + 2 is free) and stored tile kt + 1 (which the ring
            // starts reading at k-step 12).  A wave that finishes its half-tiles early does its
            // tile store and window finish while the other wave of its SIMD still multiplies.
            // The loop runs three tiles per iteration, one per key buffer, so that every LDS address in it is
            // a register plus an immediate offset.
            auto tile = [&](int kt, auto cur_c) {
                // Tile kt + 2 is loaded and stored on every iteration, past the end as a copy of the last
                // tile into the free buffer (never read): without a branch around them the compiler sees
                // each load waited for at its store and puts no wait at the loop's head, where it would
                // also wait for the previous window's candidate store to complete.
                uint4 nxt[kTileLoads];
                load_tile(kt + 2 < n_kt ? kt + 2 : n_kt - 1, nxt);
                float part_odd = 0.f, p = 0.f;
                constexpr int cur = decltype(cur_c)::value, nb = (cur + 1) % kBufs;
                const uint4 *kc = sh.keys[cur] + lane;
                const uint4 *kn = sh.keys[nb] + lane;
                // k-steps [i0, i1) of this tile
                auto steps = [&](auto i0c, auto i1c) {
                    constexpr int i0 = decltype(i0c)::value, i1 = decltype(i1c)::value;
#pragma unroll
                    for (int i = i0; i < i1; ++i) {
                        const int hf = i / 8, ks = i % 8, st = hf;
                        if (ks == 0) p = 0.f;
                        const bf16x8 b = ring[i % kRing];
                        acc[st][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][ks], b, ks == 0 ? f32x16{} : acc[st][0], 0, 0, 0);
                        acc[st][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][ks], b, ks == 0 ? f32x16{} : acc[st][1], 0, 0, 0);
                        // the ring slot just freed takes k-step i + kRing (of the next tile
                        // past the end of this one; harmless stale data after the last tile)
                        ring[i % kRing] = as_bf16x8(i + kRing < kSteps ? kc[64 * (i + kRing)] : kn[64 * (i + kRing - kSteps)]);
                        // epilogue of the previous half-tile (the other accumulator pair):
                        // register g of lane l is head 32 mt + 8 (g / 4) + 4 (l / 32) + g % 4
#pragma unroll
                        for (int g = 2 * ks; g < 2 * ks + 2; ++g) {
                            p = fmaf(wv[0][g], relu(acc[st ^ 1][0][g]), p);
                            p = fmaf(wv[1][g], relu(acc[st ^ 1][1][g]), p);
                        }
                        if (ks == 7 && hf == 0) part_odd = p;  // odd half-tile of tile kt - 1
                        step_pattern();
                    }
                };
                // The half-tiles' MFMA streams issue at raised priority: the SIMD's other wave, in its tile
                // store, window finish or selection, then issues second and the matrix pipe stays fed.
                if (selects) {
                    __builtin_amdgcn_s_setprio(1);
                    steps(std::integral_constant<int, 0>{}, std::integral_constant<int, kSteps / 2>{});
                    __builtin_amdgcn_s_setprio(0);
                }
                __syncthreads();  // every wave, selecting or not, passes it once per tile
                if (selects) {
                    __builtin_amdgcn_s_setprio(1);
                    steps(std::integral_constant<int, kSteps / 2>{}, std::integral_constant<int, kSteps>{});
                    __builtin_amdgcn_s_setprio(0);
                }
                // the next key tile goes to LDS before any candidate store is issued: its wait
                // for the key loads must not also wait for a store
                // kept after the second half's MFMAs: scheduled among them, the store would wait there for
                // the tile's loads
                __builtin_amdgcn_sched_barrier(0);
                store_tile((cur + 2) % kBufs, nxt);
                if (selects) {
                    // window: odd half-tile of tile kt - 1 and even half-tile of tile kt
                    finish_window(part_odd, p, (uint32_t)kt * kKT + lane);
                    if (!kBlockKeys && (kt % kRefresh) == kRefresh - 1 && (int64_t)kt * kKT >= m) {
                        const int b = topk::threshold_bin(hist, m, nullptr, nullptr);
                        if (b > run_bin) {
                            run_bin = b;
                            const uint32_t k_lo = (uint32_t)b << kBinShift;  // the bin's smallest key
                            run_thr = __uint_as_float((k_lo & 0x80000000u) ? (k_lo & 0x7FFFFFFFu) : ~k_lo);
                        }
                    }
                }
            };
            int kt3 = 0;
#pragma unroll 1
            for (; kt3 + kBufs <= n_kt; kt3 += kBufs) {
                tile(kt3, std::integral_constant<int, 0>{});
                tile(kt3 + 1, std::integral_constant<int, 1>{});
                tile(kt3 + 2, std::integral_constant<int, 2>{});
            }
            if (kt3 < n_kt) tile(kt3, std::integral_constant<int, 0>{});
            if (kt3 + 1 < n_kt) tile(kt3 + 1, std::integral_constant<int, 1>{});
            if (selects) {  // the odd half of the last tile
                float p = 0.f;
#pragma unroll
                for (int g = 0; g < 16; ++g) {
                    p = fmaf(wv[0][g], relu(acc[1][0][g]), p);
                    p = fmaf(wv[1][g], relu(acc[1][1][g]), p);
                }
                finish_window(p, 0.f, (uint32_t)n_kt * kKT + lane);
            }
        } else if constexpr (kBlockKeys) {
            __syncthreads();  // no barrier followed the read of sh.tile: keep it until every thread has read it
        }
        if constexpr (kBlockKeys) continue;  // no selection in this pass
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
        for (int r = 0; r < n_rows; ++r) {
            int32_t *dst = idx_all + abs_row(r) * topk;
            const int64_t pr = pos_of(r);  // the row's position
            if (pr + 1 <= topk) {  // every visible key is selected
                for (int i = tid; i < topk; i += kThreads) dst[i] = i <= pr ? i : -1;
                continue;
            }
            const int mr = topk;
            const int bin = sh.info[r][0], above = sh.info[r][1], upto = sh.info[r][2];
            const uint2 *list = cands + ((int64_t)blockIdx.x * kRows + r) * cand_ld;
            const int nl = sh.info[r][3];
            if (upto <= kCap) {
                static_assert(sizeof(RowSelScratch) <= sizeof(sh.keys), "the selection scratch fits the key tiles");
                select_row_lds((lds_sel_t *)(void *)&sh.keys[0][0], (lds_u32 *)sh.region, (lds_i32 *)(sh.region + kCap),
                               (glb_cu64 *)(const void *)list, nl, bin, above, mr, (glb_i32 *)dst);
            } else {
                topk::select_and_emit(sh.sel, topk::GlobalCands{list}, nl, bin, above, mr, dst);
            }
            for (int i = mr + tid; i < topk; i += kThreads) dst[i] = -1;
            __syncthreads();
        }
    }
}

__global__ void reset_counter_kernel(int32_t *counter) { *counter = 0; }

// Sequence b of a batch is valid when 0 <= cu[b] <= cu[b + 1] <= T and its n_b = ctx_len[b] cached tokens
// (the new ones last) satisfy cu[b + 1] - cu[b] <= n_b <= max_ctx.
__device__ __forceinline__ bool varlen_seq(const int32_t *cu, const int32_t *ctx_len, int64_t T, int32_t max_ctx,
                                           int b, int32_t *start, int32_t *len, int32_t *n)
{
    *start = cu[b];
    const int32_t end = cu[b + 1];
    *n = ctx_len[b];
    *len = end - *start;
    return *start >= 0 && *len >= 0 && end <= T && *n >= *len && *n <= max_ctx;
}

// One workgroup: the row tiles of every valid sequence, in sequence order (an exclusive scan of the
// per-sequence tile counts), then empty entries up to n_tiles.  An invalid sequence gets no tile.
// Sequences go 1024 at a time: each thread scans its sequence's tile count, then all threads write that
// block of sequences' tiles together, tile e finding its sequence by binary search over the block's
// scanned offsets.  Offsets are 64-bit and every write is bounded by n_tiles (sequences that are each
// valid may still overlap when cu_seqlens is not monotone overall).
constexpr int kVarlenThreads = 1024;
__global__ __launch_bounds__(kVarlenThreads) void varlen_tiles_kernel(
    const int32_t *__restrict__ cu, const int32_t *__restrict__ ctx_len, int32_t n_seqs, int64_t T, int32_t max_ctx,
    VarlenTile *__restrict__ tiles, int64_t n_tiles, uint32_t *err)
{
    __shared__ int wave_sums[kVarlenThreads / kWave];
    __shared__ int64_t first[kVarlenThreads + 1];  // first tile of each sequence of the block, then the end
    __shared__ VarlenTile seq_tile[kVarlenThreads];  // each sequence's tile 0 (q0 = 0)
    const int tid = threadIdx.x;
    int64_t running = 0;
#pragma unroll 1
    for (int b0 = 0; b0 < n_seqs; b0 += kVarlenThreads) {
        const int b = b0 + tid;
        int32_t start = 0, len = 0, n = 0;
        if (b < n_seqs && !varlen_seq(cu, ctx_len, T, max_ctx, b, &start, &len, &n)) {
            flag_error(err, SA_DEVERR_ROW);
            len = 0;
        }
        // a sequence of the fused path has at most max_ctx <= 524288 rows (65536 tiles): the clamp only keeps
        // the 32-bit block scan from overflowing on sizes that never reach this kernel
        const int nt = (len + kRows - 1) / kRows;
        const int ntc = nt < (1 << 20) ? nt : (1 << 20);
        int total;
        const int excl = topk::block_scan<kVarlenThreads / kWave>(ntc, wave_sums, &total);
        first[tid] = running + excl;
        if (tid == kVarlenThreads - 1) first[kVarlenThreads] = running + total;
        seq_tile[tid] = VarlenTile{b, 0, len, n - len, start, {0, 0, 0}};
        __syncthreads();
        const int64_t end = running + total < n_tiles ? running + total : n_tiles;
        for (int64_t e = running + tid; e < end; e += kVarlenThreads) {
            int lo = 0, hi = kVarlenThreads - 1;  // the last sequence with first[seq] <= e
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (first[mid] <= e) lo = mid;
                else hi = mid - 1;
            }
            VarlenTile t = seq_tile[lo];
            t.q0 = kRows * (int32_t)(e - first[lo]);
            tiles[e] = t;
        }
        running += total;
        __syncthreads();  // first / seq_tile are rewritten for the next block
    }
    for (int64_t j = running + tid; j < n_tiles; j += kVarlenThreads) tiles[j] = VarlenTile{0, 0, 0, 0, 0, {0, 0, 0}};
}

// One thread per query row r: its sequence b (cu[b] <= r < cu[b + 1], by binary search) and position
// n_b - (cu[b + 1] - cu[b]) + (r - cu[b]); a row of no valid sequence gets (-1, -1) and (idx given)
// an empty selection.
__global__ void varlen_rows_kernel(const int32_t *__restrict__ cu, const int32_t *__restrict__ ctx_len,
                                   int32_t n_seqs, int64_t T, int32_t max_ctx, int32_t topk,
                                   int32_t *__restrict__ row_seq, int32_t *__restrict__ row_pos,
                                   int32_t *__restrict__ idx, uint32_t *err)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= T) return;
    int lo = 0, hi = n_seqs - 1;  // the last b with cu[b] <= r (b = 0 if none)
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    int32_t start, len, n;
    const bool ok = varlen_seq(cu, ctx_len, T, max_ctx, lo, &start, &len, &n) && r >= start && r < start + len;
    if (!ok) {
        flag_error(err, SA_DEVERR_ROW);
        if (idx)
            for (int i = 0; i < topk; ++i) idx[r * topk + i] = -1;
    }
    row_seq[r] = ok ? lo : -1;
    row_pos[r] = ok ? n - len + (int32_t)(r - start) : -1;
}

// Query rows that each name their sequence and position, cut into row tiles of one sequence: one workgroup
// sorts the T <= kRowTileMaxRows rows by (sequence, position, row) -- a 64-bit key per row in LDS, bitonic
// sort -- and cuts each sequence's run of the sorted order into tiles of 8 rows; tiles past the last get
// n = 0.  A row whose sequence or position is out of range sets SA_DEVERR_ROW, sorts last, belongs to no
// tile and gets an empty index list.  Key: sequence (31 bits) | position (19 bits) | row (14 bits).
constexpr int kRowTileMaxRows = 16384;
constexpr int kRowTileThreads = 1024;
constexpr int kRowTilePer = kRowTileMaxRows / kRowTileThreads;  // sorted entries per thread in the cut (16)
constexpr uint64_t kNoKey = ~0ull;

__global__ __launch_bounds__(kRowTileThreads) void row_tiles_kernel(
    const int32_t *__restrict__ row_seq, const int32_t *__restrict__ row_pos, int32_t T, int32_t n_seqs,
    int32_t max_ctx, int32_t topk, RowTile *__restrict__ tiles, int32_t n_tiles, int32_t *__restrict__ idx,
    uint32_t *err)
{
    __shared__ uint64_t key[kRowTileMaxRows];
    __shared__ int scan[kRowTileThreads];
    __shared__ int wave_sums[kRowTileThreads / kWave];
    const int tid = threadIdx.x;
    int N = 2;
    while (N < T) N *= 2;
    for (int i = tid; i < N; i += kRowTileThreads) {
        uint64_t k = kNoKey;
        if (i < T) {
            const int32_t b = row_seq[i], p = row_pos[i];
            if (b >= 0 && b < n_seqs && p >= 0 && p < max_ctx) {
                k = ((uint64_t)b << 33) | ((uint64_t)p << 14) | (uint64_t)i;
            } else {
                flag_error(err, SA_DEVERR_ROW);
                for (int j = 0; j < topk; ++j) idx[(int64_t)i * topk + j] = -1;
            }
        }
        key[i] = k;
    }
    __syncthreads();
    // bitonic sort, ascending
    for (int k = 2; k <= N; k *= 2) {
        for (int j = k / 2; j > 0; j /= 2) {
            for (int i = tid; i < N; i += kRowTileThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t a = key[i], c = key[ixj];
                    if ((a > c) == ((i & k) == 0)) {
                        key[i] = c;
                        key[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    // cut: thread c takes sorted entries [16 c, 16 c + 16).  Entry i starts a tile when its offset from the
    // start of its sequence's run is a multiple of 8; tile of entry i = tile starts up to i, minus one.
    const int i0 = tid * kRowTilePer;
    const auto seq_of = [&](int i) { return (int)(key[i] >> 33); };
    const auto valid = [&](int i) { return i < N && key[i] != kNoKey; };
    int last_start = -1;  // last run start in this thread's entries
    for (int u = 0; u < kRowTilePer; ++u) {
        const int i = i0 + u;
        if (valid(i) && (i == 0 || seq_of(i - 1) != seq_of(i))) last_start = i;
    }
    // inclusive max-scan of the run starts over the threads (Hillis-Steele), then this thread's carry
    scan[tid] = last_start;
    __syncthreads();
    for (int d = 1; d < kRowTileThreads; d *= 2) {
        const int v = tid >= d ? scan[tid - d] : -1;
        __syncthreads();
        if (v > scan[tid]) scan[tid] = v;
        __syncthreads();
    }
    int begin = tid > 0 ? scan[tid - 1] : -1;  // run start before this thread's entries
    int starts = 0;
    for (int u = 0; u < kRowTilePer; ++u) {
        const int i = i0 + u;
        if (!valid(i)) break;
        if (i == 0 || seq_of(i - 1) != seq_of(i)) begin = i;
        starts += ((i - begin) % kRows) == 0 ? 1 : 0;
    }
    int n_total;
    int tile = topk::block_scan<kRowTileThreads / kWave>(starts, wave_sums, &n_total) - 1;
    begin = tid > 0 ? scan[tid - 1] : -1;
    for (int u = 0; u < kRowTilePer; ++u) {
        const int i = i0 + u;
        if (!valid(i)) break;
        const int sq = seq_of(i);
        if (i == 0 || seq_of(i - 1) != sq) begin = i;
        const int slot = (i - begin) % kRows;
        if (slot == 0) ++tile;
        if (tile >= n_tiles) break;  // cannot happen: n_tiles bounds the tiles of T rows
        RowTile &t = tiles[tile];
        t.row[slot] = (int32_t)(key[i] & 0x3FFF);
        t.pos[slot] = (int32_t)((key[i] >> 14) & 0x7FFFF);
        if (slot == 0) t.seq = sq;
        const bool last = slot == kRows - 1 || !valid(i + 1) || seq_of(i + 1) != sq;
        if (last) t.n = slot + 1;
    }
    for (int e = n_total + tid; e < n_tiles; e += kRowTileThreads) {
        tiles[e].seq = 0;
        tiles[e].n = 0;
    }
}

}  // namespace

size_t prefill_block_keys_ld(int64_t L, int64_t pos0) { return (pos0 + L + kKT - 1) / kKT; }

size_t prefill_topk_workspace(const sa_handle_s &h, int64_t L, int64_t pos0)
{
    const int64_t n_tiles = (L + kRows - 1) / kRows;
    const int64_t slots = n_tiles < h.n_cu ? n_tiles : h.n_cu;
    const int64_t ld = (pos0 + L + 63) / 64 * 64;  // a candidate list holds at most every key
    return 256 + (size_t)slots * kRows * (size_t)ld * sizeof(uint2);
}

// Capacity for T rows (any number of sequences: at most min(n_seqs, T) of them own rows):
// [counter | candidate lists of the workgroup slots | tile table]
struct VarlenLayout {
    int64_t tiles_cap, slots_cap, ld;
    size_t cands, tiles, total;
};
VarlenLayout varlen_layout(const sa_handle_s &h, int64_t T, int32_t max_ctx)
{
    VarlenLayout v;
    v.tiles_cap = (T + kRows - 1) / kRows + T;
    v.slots_cap = v.tiles_cap < h.n_cu ? v.tiles_cap : h.n_cu;
    v.ld = ((int64_t)max_ctx + 63) / 64 * 64;  // a candidate list holds at most every key
    v.cands = 256;
    v.tiles = v.cands + (size_t)v.slots_cap * kRows * (size_t)v.ld * sizeof(uint2);
    v.total = v.tiles + (size_t)v.tiles_cap * sizeof(VarlenTile);
    return v;
}

size_t prefill_varlen_workspace(const sa_handle_s &h, int64_t T, int32_t max_ctx)
{
    return varlen_layout(h, T, max_ctx).total;
}

hipError_t launch_varlen_rows(sa_handle_s &h, const int32_t *cu, const int32_t *ctx_len, int32_t n_seqs, int64_t T,
                              int32_t max_ctx, int32_t topk, int32_t *idx, int32_t *row_seq, int32_t *row_pos,
                              hipStream_t st)
{
    hipLaunchKernelGGL(varlen_rows_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, cu, ctx_len, n_seqs, T,
                       max_ctx, topk, row_seq, row_pos, idx, h.d_err);
    return hipGetLastError();
}

hipError_t launch_prefill_varlen(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                                 int64_t n_pages, const int32_t *block_table, int32_t max_blocks, const int32_t *cu,
                                 const int32_t *ctx_len, int32_t n_seqs, int64_t T, int32_t max_ctx, int32_t topk,
                                 int32_t *idx, void *ws, hipStream_t st)
{
    const VarlenLayout v = varlen_layout(h, T, max_ctx);
    const int64_t n_tiles = (T + kRows - 1) / kRows + (n_seqs < T ? n_seqs : T);
    const int64_t slots = n_tiles < h.n_cu ? n_tiles : h.n_cu;
    char *base = reinterpret_cast<char *>(ws);
    int32_t *counter = reinterpret_cast<int32_t *>(base);
    uint2 *cands = reinterpret_cast<uint2 *>(base + v.cands);
    VarlenTile *tiles = reinterpret_cast<VarlenTile *>(base + v.tiles);
    hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(1), 0, st, counter);
    hipLaunchKernelGGL(varlen_tiles_kernel, dim3(1), dim3(kVarlenThreads), 0, st, cu, ctx_len, n_seqs, T, max_ctx,
                       tiles, n_tiles, h.d_err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    KeySource ks{reinterpret_cast<const uint16_t *>(kidx_pages), block_table, n_pages, h.d_err};
    ks.tiles = tiles;
    ks.table_ld = max_blocks;
    const BlockKeysOut none{nullptr, 0};
    KernelTimer timer(h, SA_KERNEL_INDEXER, st);
    hipLaunchKernelGGL((indexer_topk_prefill_kernel<true, false>), dim3((unsigned)slots), dim3(kThreads), 0, st,
                       reinterpret_cast<const uint16_t *>(q_idx), w, ks, (int64_t)0, (int64_t)0, topk, (int64_t)topk,
                       idx, cands, v.ld, none, counter, (int32_t)n_tiles);
    return hipGetLastError();
}

// Rows naming their own (sequence, position): [counter | candidate lists of the workgroup slots | row table]
struct RowsLayout {
    int64_t tiles_cap, slots, ld;
    size_t cands, table, total;
};
RowsLayout rows_layout(const sa_handle_s &h, int64_t T, int32_t max_ctx)
{
    RowsLayout r;
    r.tiles_cap = T;  // never more tiles than rows (one row per tile when every row has its own sequence)
    r.slots = r.tiles_cap < h.n_cu ? r.tiles_cap : h.n_cu;
    r.ld = ((int64_t)max_ctx + 63) / 64 * 64;
    r.cands = 256;
    r.table = r.cands + (size_t)r.slots * kRows * (size_t)r.ld * sizeof(uint2);
    r.total = r.table + (size_t)r.tiles_cap * sizeof(RowTile);
    return r;
}

bool prefill_rows_fused(const sa_handle_s &h, int64_t T, int32_t max_ctx)
{
    static_assert(kPrefillMaxPages * 64 <= (1 << 19), "positions take 19 bits of the sort key");
    return h.fast_decode && T <= kRowTileMaxRows && ((int64_t)max_ctx + 63) / 64 <= kPrefillMaxPages;
}

size_t prefill_rows_workspace(const sa_handle_s &h, int64_t T, int32_t max_ctx)
{
    return rows_layout(h, T, max_ctx).total;
}

hipError_t launch_prefill_rows(sa_handle_s &h, const void *q_idx, const float *w, const void *kidx_pages,
                               int64_t n_pages, const int32_t *block_table, int32_t max_blocks, const int32_t *row_seq,
                               const int32_t *row_pos, int32_t n_seqs, int64_t T, int32_t max_ctx, int32_t topk,
                               int32_t *idx, void *ws, hipStream_t st)
{
    const RowsLayout r = rows_layout(h, T, max_ctx);
    char *base = reinterpret_cast<char *>(ws);
    int32_t *counter = reinterpret_cast<int32_t *>(base);
    uint2 *cands = reinterpret_cast<uint2 *>(base + r.cands);
    RowTile *tiles = reinterpret_cast<RowTile *>(base + r.table);
    hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(1), 0, st, counter);
    hipLaunchKernelGGL(row_tiles_kernel, dim3(1), dim3(kRowTileThreads), 0, st, row_seq, row_pos, (int32_t)T, n_seqs,
                       max_ctx, topk, tiles, (int32_t)r.tiles_cap, idx, h.d_err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    KeySource ks{reinterpret_cast<const uint16_t *>(kidx_pages), block_table, n_pages, h.d_err};
    ks.rows = tiles;
    ks.table_ld = max_blocks;
    const BlockKeysOut none{nullptr, 0};
    KernelTimer timer(h, SA_KERNEL_INDEXER, st);
    hipLaunchKernelGGL((indexer_topk_prefill_kernel<true, false>), dim3((unsigned)r.slots), dim3(kThreads), 0, st,
                       reinterpret_cast<const uint16_t *>(q_idx), w, ks, (int64_t)0, (int64_t)0, topk, (int64_t)topk,
                       idx, cands, r.ld, none, counter, (int32_t)r.tiles_cap);
    return hipGetLastError();
}

hipError_t launch_prefill_topk(sa_handle_s &h, const void *q_idx, const float *w, const void *k_idx,
                               int64_t L, int32_t topk, int32_t *idx, void *ws, hipStream_t st,
                               const int32_t *table, int64_t n_pages, int64_t pos0, uint32_t *block_keys,
                               int64_t keys_above)
{
    const int64_t n_tiles = (L + kRows - 1) / kRows;
    const int64_t slots = n_tiles < h.n_cu ? n_tiles : h.n_cu;
    const int64_t ld = (pos0 + L + 63) / 64 * 64;
    int32_t *counter = reinterpret_cast<int32_t *>(ws);
    uint2 *cands = reinterpret_cast<uint2 *>(reinterpret_cast<char *>(ws) + 256);
    hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(1), 0, st, counter);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const KeySource ks{reinterpret_cast<const uint16_t *>(k_idx), table, n_pages, h.d_err};
    const uint16_t *qi = reinterpret_cast<const uint16_t *>(q_idx);
    KernelTimer timer(h, SA_KERNEL_INDEXER, st);
    if (block_keys) {
        const BlockKeysOut bk{block_keys, (int64_t)prefill_block_keys_ld(L, pos0)};
        const int64_t need = keys_above;
        if (table)
            hipLaunchKernelGGL((indexer_topk_prefill_kernel<true, true>), dim3((unsigned)slots), dim3(kThreads), 0, st,
                               qi, w, ks, L, pos0, topk, need, idx, cands, ld, bk, counter, (int32_t)n_tiles);
        else
            hipLaunchKernelGGL((indexer_topk_prefill_kernel<false, true>), dim3((unsigned)slots), dim3(kThreads), 0,
                               st, qi, w, ks, L, pos0, topk, need, idx, cands, ld, bk, counter, (int32_t)n_tiles);
        return hipGetLastError();
    }
    const BlockKeysOut none{nullptr, 0};
    if (table)
        hipLaunchKernelGGL((indexer_topk_prefill_kernel<true, false>), dim3((unsigned)slots), dim3(kThreads), 0, st,
                           qi, w, ks, L, pos0, topk, (int64_t)topk, idx, cands, ld, none, counter, (int32_t)n_tiles);
    else
        hipLaunchKernelGGL((indexer_topk_prefill_kernel<false, false>), dim3((unsigned)slots), dim3(kThreads), 0, st,
                           qi, w, ks, L, pos0, topk, (int64_t)topk, idx, cands, ld, none, counter, (int32_t)n_tiles);
    return hipGetLastError();
}

}  // namespace sa
