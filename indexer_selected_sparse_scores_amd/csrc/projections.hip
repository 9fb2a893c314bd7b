// Index-space projections on gfx950: the first two lines of the pseudocode in "Sparse Attention
// and RL Optimization: Three Technical Breakthroughs in LLM Post-Training", section 2.5 -- the
// index query and key are linear maps of the attention query and key (i_q = W_iq(q),
// i_k = W_ik(k)).  The head weights w(t, j) of the score in section 2.2 are taken as one more
// linear map of the query row.
//
//  * q side: q_idx = q W_iq^T (bf16 out) and w = q W_w^T (fp32 out), one kernel and one pass over
//    the H * d_qk query rows (9216 wide for the latent shapes): [W_iq; W_w] is the B operand of a
//    tiled bf16 GEMM on v_mfma_f32_32x32x16_bf16 with fp32 accumulation, whose last column tile is
//    the head weights'.
//  * k side: k_idx = k W_ik^T over the 576-wide latent row on v_mfma_f32_32x32x16_bf16, W_ik
//    held in LDS by persistent workgroups, each projected row written straight to where it
//    belongs: the contiguous [L, d_I] array, or the token's slot of the paged index-key cache.
#include <string>
#include <type_traits>

#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

namespace {

constexpr int kPD = 128;                 // index dims (d_I) of the key projection kernel
constexpr int kPWaves = 8;                // two waves per SIMD
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPRows = 32;               // tokens per wave tile

// Destination of projected key row r (a lane's token; r < L): the contiguous [L, d_I] array, or
// page block_table[seq, pos / page_size], slot pos % page_size with (seq, pos) = (row_seq[r],
// row_pos[r]), defaulting to (0, pos0 + r); nullptr when any part is out of range (the caller
// flags it).  The block-table load is made for every lane, at a clamped index, so that no load
// sits behind a lane-dependent branch.
template <bool PAGED>
__device__ __forceinline__ uint16_t *key_row_dst(int64_t r, uint16_t *out, const int32_t *block_table, int32_t n_seqs,
                                                 int32_t max_blocks, int32_t page_size, int64_t n_pages,
                                                 const int32_t *row_seq, const int32_t *row_pos, int64_t pos0)
{
    if (!PAGED) return out + r * kPD;
    const int64_t seq = row_seq ? row_seq[r] : 0;
    const int64_t pos = row_pos ? (int64_t)row_pos[r] : pos0 + r;
    const int64_t lp = pos >= 0 ? pos / page_size : -1;
    const bool ok = lp >= 0 && lp < max_blocks && seq >= 0 && seq < n_seqs;
    const int32_t page = block_table[ok ? seq * max_blocks + lp : 0];
    if (!ok || page < 0 || page >= n_pages) return nullptr;
    return out + ((int64_t)page * page_size + pos % page_size) * kPD;
}

// Persistent: each workgroup copies W_ik once into LDS, in MFMA B-fragment order (fragment
// (nt, s) = index dims 32 nt .. +31, k-elements 16 s .. +15, one linear 1 KB block: lane l holds
// dim 32 nt + l % 32, elements 16 s + 8 (l / 32) .. +7), then its waves take 32-token tiles in
// turn.  A wave multiplies its tile's rows by all 128 index dims (four 32x32 accumulators).  Its
// A fragments (token l % 32, elements 16 s + 8 (l / 32) .. +7) stream through a ring of KD
// k-steps of registers: the load for k-step s + KD (of this tile, or of the wave's next tile) is
// issued as soon as k-step s's products are, so KD KB per wave stay in flight across tiles; the
// B fragments are read from LDS one k-step ahead.  The fp32 results are rounded to bf16 and each
// row is stored where it belongs.
template <int KS, bool PAGED>  // K / 16 k-steps; destination in the paged cache or contiguous
__global__ __launch_bounds__(kPThreads, 1) void project_k_kernel(
    const uint16_t *__restrict__ k, int64_t L, const uint16_t *__restrict__ W, uint16_t *__restrict__ out,
    const int32_t *__restrict__ block_table, int32_t n_seqs, int32_t max_blocks, int32_t page_size, int64_t n_pages,
    const int32_t *__restrict__ row_seq, const int32_t *__restrict__ row_pos, int64_t pos0, uint32_t *err)
{
    constexpr int K = 16 * KS;
    constexpr int KD = KS >= 16 ? KS / 2 : KS;  // ring depth in k-steps; divides KS
    static_assert(KS % KD == 0, "a tile must fill the ring a whole number of times");
    typedef __attribute__((address_space(1))) uint32_t global_u32;
    extern __shared__ __attribute__((aligned(16))) uint4 wfrag[];  // 4 KS fragments of 64 x 16 bytes
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    for (int f = wave; f < 4 * KS; f += kPWaves) {
        const int nt = f / KS, st = f % KS;
        wfrag[f * kWave + lane] = load16(W + (int64_t)(32 * nt + lane % 32) * K + 16 * st + 8 * (lane / 32));
    }
    __syncthreads();

    const int64_t n_tiles = (L + kPRows - 1) / kPRows;
    const int64_t stride = (int64_t)gridDim.x * kPWaves;
    // token rows are clamped into [0, L): a tile past the end loads row L - 1 and is never used
    auto a_ptr = [&](int64_t tile) {
        int64_t arow = tile * kPRows + lane % 32;
        if (arow >= L) arow = L - 1;
        return k + arow * (int64_t)K + 8 * (lane / 32);
    };
    bf16x8 a[KD];
    int64_t tile = (int64_t)blockIdx.x * kPWaves + wave;
    const uint16_t *cp = a_ptr(tile);
#pragma unroll
    for (int s = 0; s < KD; ++s) {
        a[s] = as_bf16x8(load16(cp + 16 * s));
        __builtin_amdgcn_sched_barrier(0);  // issued in k-step order, the order the loop consumes them
    }
    const bool odd = lane & 1;
    for (; tile < n_tiles; tile += stride) {
        const int64_t r0 = tile * kPRows;
        const bool mine = r0 + lane % 32 < L;
        // every lane resolves its token's destination (the lanes of both halves alike) before the
        // products, so the loads involved are long done by the stores
        uint16_t *my_dst = key_row_dst<PAGED>(mine ? r0 + lane % 32 : L - 1, out, block_table, n_seqs, max_blocks,
                                              page_size, n_pages, row_seq, row_pos, pos0);
        const uint16_t *np = a_ptr(tile + stride);
        // opaque per tile, so the fragment reads (the same every tile) are not hoisted out of the loop
        int wl = lane;
        asm volatile("" : "+v"(wl));
        f32x16 acc[4] = {};
        uint4 b[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) b[nt] = wfrag[(nt * KS) * kWave + wl];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 bn[4];
            if (s + 1 < KS) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) bn[nt] = wfrag[(nt * KS + s + 1) * kWave + wl];
            }
            const bf16x8 cur = a[s % KD];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, as_bf16x8(b[nt]), acc[nt], 0, 0, 0);
            a[s % KD] = as_bf16x8(load16(s + KD < KS ? cp + 16 * (s + KD) : np + 16 * (s + KD - KS)));
            if (s + 1 < KS) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) b[nt] = bn[nt];
            }
            __builtin_amdgcn_sched_barrier(0);  // keep each k-step's refill where it is issued
        }
        cp = np;
        if (PAGED && mine && lane < kPRows && !my_dst) flag_error(err, SA_DEVERR_BLOCK_TABLE);
        if (!mine) my_dst = nullptr;
        // register i of lane l: token r0 + 8 (i / 4) + 4 (l / 32) + i % 4, index dim 32 nt + l % 32.
        // Lane j < 32 holds the destination of token r0 + j, shared through the wave.
        const uint64_t my_bits = reinterpret_cast<uint64_t>(my_dst);
        // Registers i and i + 1 hold consecutive tokens.  Neighbouring lanes swap one of them so that
        // an even lane stores dims (d, d + 1) of the first token and an odd lane those of the second,
        // as one 4-byte store each.
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const int tr = 8 * (i / 4) + 4 * (lane / 32) + i % 4 + (odd ? 1 : 0);
            const uint64_t dst = ((uint64_t)__shfl((uint32_t)(my_bits >> 32), tr) << 32) | __shfl((uint32_t)my_bits, tr);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float give = odd ? acc[nt][i] : acc[nt][i + 1];
                const float got = __builtin_bit_cast(
                    float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, give), 0xB1, 0xF, 0xF, false));  // lane ^ 1
                const float d0 = odd ? got : acc[nt][i], d1 = odd ? acc[nt][i + 1] : got;
                const uint32_t v = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)d0) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)d1) << 16);
                if (dst) *(global_u32 *)(dst + 2 * (32 * nt + (lane % 32 & ~1))) = v;
            }
        }
    }
}

// ---- query side -----------------------------------------------------------------------------
// One workgroup of eight waves (two per SIMD, so that one wave's LDS and memory waits are covered by the
// other's products) computes a 256 x 256 tile of [q_idx | w] = q [W_iq; W_w]^T: wave (wm, wn), wm = 0..1,
// wn = 0..3, its 128 x 64 part as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16.  K advances in blocks of 64
// through two LDS buffers, each holding the block's 256 A rows and 256 B rows row-major (128 bytes a row)
// with the eight 16-byte chunks of row r permuted to position c ^ swz(r), so the operand reads (32 rows of
// one chunk per half-wave) hit distinct banks.  Each wave moves 64 of the rows: 8 loads of 8 whole rows (1 KB,
// eight 128-byte lines) per block into registers and, three k-steps later, into the block's buffer, two loads
// and two stores beside the 8 products of every k-step.  The one barrier per block comes before its last
// k-step: it publishes the next block and frees the buffer just read.  Workgroups are ordered by XCD (id % 8):
// each XCD takes its own M tiles, kQGroupM at a time with every N tile, so its concurrent workgroups share
// their q and weight blocks through its L2.  The column tile past W_iq's is W_w's (n_w <= 256 rows, fp32 out).
constexpr int kQM = 256, kQN = 256, kQK = 64;     // workgroup tile and K block
constexpr int kQWaves = 8;
constexpr int kQThreads = kQWaves * kWave;
constexpr int kQPanelBytes = kQM * kQK * 2;       // one operand's rows of a K block: 32 KB
constexpr int kQBufBytes = 2 * kQPanelBytes;      // A and B: 64 KB
constexpr int kQLdsBytes = 2 * kQBufBytes;        // two buffers
constexpr int kQLoads = 2 * kQM / 8 / kQWaves;     // 8-row loads per wave per K block (8)
constexpr int kQGroupM = 4;                        // M tiles an XCD works on at once
constexpr int kXcds = 8;

struct ProjQArgs {
    const uint16_t *q, *w_iq, *w_w;
    uint16_t *q_idx;
    float *w;
    int64_t M;        // query rows
    int K;            // row width (multiple of 64)
    int n_iq_tiles;   // column tiles of W_iq (N1 / 256; 0 without W_iq)
    int n_w;          // rows of W_w (0 without it)
    int n_n;          // column tiles in all
    int64_t n_m;      // row tiles
};

// chunk permutation of a row: a bijection on each 8 rows, and on the even (odd) rows of each 16, so the
// 8 or 16 lanes an LDS cycle serves read distinct banks
__device__ __forceinline__ int qswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__global__ __launch_bounds__(kQThreads, 1) void project_q_kernel(ProjQArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char qlds[];  // two K-block buffers
    typedef __attribute__((address_space(1))) uint32_t global_u32;
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int id = blockIdx.x, xcd = id % kXcds, j = id / kXcds;
    const int per_group = kQGroupM * a.n_n;
    const int64_t mt = ((int64_t)(j / per_group) * kQGroupM + (j % per_group) % kQGroupM) * kXcds + xcd;
    const int nt = (j % per_group) / kQGroupM;
    if (mt >= a.n_m) return;
    const bool w_tile = nt >= a.n_iq_tiles;
    const int64_t m0 = mt * kQM;
    const int64_t K = a.K;

    // this wave's rows: waves 0..3 the A rows 64 wave + 8 jl + l / 8, waves 4..7 the B rows 64 (wave - 4) +
    // 8 jl + l / 8 (jl = 0 .. 7); lane l takes chunk (l % 8) ^ swz(row) of its row.  Rows past M or past
    // W_w's n_w rows are clamped: loaded but never stored.
    const uint16_t *gp[kQLoads];
#pragma unroll
    for (int jl = 0; jl < kQLoads; ++jl) {
        const int r = 64 * (wave & 3) + 8 * jl + lane / 8;
        const int c = (lane & 7) ^ qswz(r);
        int64_t row;
        const uint16_t *base;
        if (wave < 4) {
            row = m0 + r < a.M ? m0 + r : a.M - 1;
            base = a.q;
        } else if (w_tile) {
            row = r < a.n_w ? r : a.n_w - 1;
            base = a.w_w;
        } else {
            row = (int64_t)nt * kQN + r;
            base = a.w_iq;
        }
        gp[jl] = base + row * K + 8 * c;
    }
    // staged rows: load jl of a block goes to stg[jl] and from there to LDS bytes 1024 jl + 16 l of the wave's
    // 8 KB of the block's buffer (position l % 8 of row 8 jl + l / 8 of the wave's 64)
    uint4 stg[kQLoads];
    unsigned char *const dst0 = qlds + (wave < 4 ? 0 : kQPanelBytes) + 8192 * (wave & 3) + 16 * lane;
    auto load = [&](int kb, int jl) { stg[jl] = load16(gp[jl] + (int64_t)kb * kQK); };
    auto store = [&](int jl, int buf) {
        *reinterpret_cast<uint4 *>(dst0 + buf * kQBufBytes + 1024 * jl) = stg[jl];
    };

    const int wm = wave >> 2, wn = wave & 3;
    // operand reads: lane l reads row 32 i + l % 32 of its wave's rows, chunk 2 s + l / 32 of k-step s, which
    // sits at position (2 s) ^ y with y = (l / 32) ^ swz(l % 32)
    const int y = (lane >> 5) ^ qswz(lane & 31);
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(qlds) + 128u * (lane & 31);
    uint32_t ra0[4], rb0[4];  // buffer-0 addresses of k-steps 0..3
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        const uint32_t c = (uint32_t)(((2 * s2) ^ y) << 4);
        ra0[s2] = lds0 + 16384u * wm + c;
        rb0[s2] = lds0 + kQPanelBytes + 8192u * wn + c;
    }
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) acc[i][jn] = f32x16{};

    // fragments of one k-step: A rows 32 i + l % 32 (i = 0..3), B rows 32 jn + l % 32 (jn = 0..1)
    auto read_step = [&](int kb, int s2, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
        const uint32_t off = (uint32_t)((kb & 1) * kQBufBytes);
        const uint32_t pa = ra0[s2] + off, pb = rb0[s2] + off;
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fa[i]) : "v"(pa), "i"(4096 * i) : "memory");
#pragma unroll
        for (int i = 0; i < 2; ++i) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fb[i]) : "v"(pb), "i"(4096 * i) : "memory");
    };
    auto wait_lds = [](int n, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {  // n: 6 or 0 reads may stay in flight
        if (n == 6)
            asm volatile("s_waitcnt lgkmcnt(6)"
                         : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1])
                         :
                         : "memory");
        else
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1])
                         :
                         : "memory");
    };
    // the 8 products of one k-step, with the stores of staged group sg (rows jl = 2 sg, 2 sg + 1) to buffer buf
    // after products 0 and 1 and the loads of group lg of block kb into the same registers after products 2
    // and 3 (lg != sg)
    auto step = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[2], int sg, int buf, int lg, int kb) {
        __builtin_amdgcn_s_setprio(1);  // the SIMD's other wave, waiting on LDS or memory, issues second
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jn = 0; jn < 2; ++jn) {
                const int n = 2 * i + jn;
                acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[jn], acc[i][jn], 0, 0, 0);
                if (n < 2)
                    store(2 * sg + n, buf);
                else if (n < 4)
                    load(kb, 2 * lg + n - 2);
                __builtin_amdgcn_sched_barrier(0);
            }
        __builtin_amdgcn_s_setprio(0);
    };

    const int n_kb = a.K / kQK;
    // The staging registers are a ring of four groups of two loads: group g of a block is loaded at k-step g
    // and stored three k-steps later, so each k-step of block kb stores one group of block kb + 1 (k-steps
    // 0..2: groups 1..3) or of block kb + 2 (k-step 3: group 0, into the buffer the barrier has just freed)
    // and loads group g of block kb + 2.  At the start of iteration kb buffer kb % 2 holds block kb and buffer
    // (kb + 1) % 2 group 0 of block kb + 1, its groups 1..3 staged.  Past the end the loads repeat the last
    // block (stored to a free buffer, never used), so the loop has no branch.
    auto last = [&](int kb) { return kb < n_kb ? kb : n_kb - 1; };
#pragma unroll
    for (int jl = 0; jl < kQLoads; ++jl) load(0, jl);
#pragma unroll
    for (int jl = 0; jl < kQLoads; ++jl) store(jl, 0);
#pragma unroll
    for (int jl = 0; jl < kQLoads; ++jl) load(last(1), jl);
#pragma unroll
    for (int jl = 0; jl < 2; ++jl) store(jl, 1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    bf16x8 f0a[4], f0b[2], f1a[4], f1b[2];
    read_step(0, 0, f0a, f0b);
#pragma unroll 1
    for (int kb = 0; kb < n_kb; ++kb) {
        const int nb = (kb + 1) & 1, kl = last(kb + 2);
        read_step(kb, 1, f1a, f1b);
        wait_lds(6, f0a, f0b);
        step(f0a, f0b, 1, nb, 0, kl);
        read_step(kb, 2, f0a, f0b);
        wait_lds(6, f1a, f1b);
        step(f1a, f1b, 2, nb, 1, kl);
        read_step(kb, 3, f1a, f1b);
        wait_lds(6, f0a, f0b);
        step(f0a, f0b, 3, nb, 2, kl);
        // every wave's reads of block kb and stores of block kb + 1 are done: after the barrier block kb + 1 is
        // read and buffer kb % 2 takes block kb + 2
        wait_lds(0, f1a, f1b);
        asm volatile("s_barrier" ::: "memory");
        read_step(last(kb + 1), 0, f0a, f0b);
        step(f1a, f1b, 0, kb & 1, 3, kl);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    // register r of lane l in accumulator (i, jn): row 128 wm + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4, column
    // 64 wn + 32 jn + l % 32 of the tile
    const bool odd = lane & 1;
    const int64_t rbase = m0 + 128 * wm + 4 * (lane / 32);
    if (!w_tile) {
        // bf16: neighbouring lanes swap one of two consecutive rows, so that each lane stores two adjacent
        // columns of one row as one 4-byte store
        const int64_t col0 = (int64_t)nt * kQN + 64 * wn + (lane % 32 & ~1);
        const int64_t ldo = (int64_t)a.n_iq_tiles * kQN;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int64_t row = rbase + 32 * i + 8 * (r / 4) + r % 4 + (odd ? 1 : 0);
#pragma unroll
                for (int jn = 0; jn < 2; ++jn) {
                    const float give = odd ? acc[i][jn][r] : acc[i][jn][r + 1];
                    const float got = __builtin_bit_cast(
                        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, give), 0xB1, 0xF, 0xF, false));  // lane ^ 1
                    const float d0 = odd ? got : acc[i][jn][r], d1 = odd ? acc[i][jn][r + 1] : got;
                    const uint32_t v = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)d0) |
                                       ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)d1) << 16);
                    if (row < a.M) *(global_u32 *)(a.q_idx + row * ldo + col0 + 32 * jn) = v;
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = rbase + 32 * i + 8 * (r / 4) + r % 4;
#pragma unroll
                for (int jn = 0; jn < 2; ++jn) {
                    const int col = 64 * wn + 32 * jn + lane % 32;
                    if (row < a.M && col < a.n_w) a.w[row * a.n_w + col] = acc[i][jn][r];
                }
            }
    }
}

}  // namespace

size_t projection_workspace() { return 0; }

sa_status_t launch_project_q(sa_handle_s &h, const void *q, int64_t L, const void *W_iq, const void *W_w,
                             void *q_idx, float *w, void *ws, size_t ws_bytes, hipStream_t st)
{
    (void)ws;
    (void)ws_bytes;
    // shapes checked by the caller: K a multiple of 64, N1 of 256, n_w <= 256
    const int64_t K = (int64_t)h.cfg.n_heads * h.cfg.d_qk;
    const int64_t N1 = W_iq ? (int64_t)h.cfg.n_idx_heads * h.cfg.d_idx : 0;
    const int n_w = W_w ? h.cfg.n_idx_heads : 0;
    ProjQArgs a{reinterpret_cast<const uint16_t *>(q), reinterpret_cast<const uint16_t *>(W_iq),
                reinterpret_cast<const uint16_t *>(W_w), reinterpret_cast<uint16_t *>(q_idx), w, L, (int)K,
                (int)(N1 / kQN), n_w, (int)(N1 / kQN) + (n_w > 0 ? 1 : 0), (L + kQM - 1) / kQM};
    // workgroups: per XCD, groups of kQGroupM row tiles times every column tile
    const int64_t groups = (a.n_m + (int64_t)kQGroupM * kXcds - 1) / ((int64_t)kQGroupM * kXcds);
    const int64_t grid = groups * kQGroupM * a.n_n * kXcds;
    if (grid > INT32_MAX) {
        h.last_error = "too many query rows for one launch";
        return SA_ERR_UNSUPPORTED;
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(project_q_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kQLdsBytes);
    if (e == hipSuccess) {
        KernelTimer timer(h, SA_KERNEL_PROJECT, st);
        hipLaunchKernelGGL(project_q_kernel, dim3((unsigned)grid), dim3(kQThreads), kQLdsBytes, st, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        h.last_error = std::string("query projection launch: ") + hipGetErrorString(e);
        return SA_ERR_HIP;
    }
    return SA_OK;
}

hipError_t launch_project_k(sa_handle_s &h, const void *k, int64_t L, const void *W_ik, void *k_idx,
                            const int32_t *block_table, int32_t n_seqs, int32_t max_blocks, int64_t n_pages,
                            const int32_t *row_seq, const int32_t *row_pos, int64_t pos0, hipStream_t st)
{
    const int K = h.cfg.n_kv_heads * h.cfg.d_qk;
    const int64_t n_tiles = (L + kPRows - 1) / kPRows;
    const int64_t want = (n_tiles + kPWaves - 1) / kPWaves;
    const unsigned grid = (unsigned)(want < h.n_cu ? want : h.n_cu);
    // one instantiation per supported key-row width (k-steps of 16 elements)
    auto run = [&](auto ks_c) -> hipError_t {
        constexpr int KS = decltype(ks_c)::value;
        const size_t lds = (size_t)4 * KS * kWave * 16;  // W_ik as B fragments
        const void *fn = block_table ? reinterpret_cast<const void *>(project_k_kernel<KS, true>)
                                     : reinterpret_cast<const void *>(project_k_kernel<KS, false>);
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        KernelTimer timer(h, SA_KERNEL_PROJECT, st);
        hipLaunchKernelGGL((block_table ? project_k_kernel<KS, true> : project_k_kernel<KS, false>), dim3(grid),
                           dim3(kPThreads), lds, st,
                           reinterpret_cast<const uint16_t *>(k), L, reinterpret_cast<const uint16_t *>(W_ik),
                           reinterpret_cast<uint16_t *>(k_idx), block_table, n_seqs, max_blocks, h.cfg.page_size,
                           n_pages, row_seq, row_pos, pos0, h.d_err);
        return hipGetLastError();
    };
    switch (K) {
    case 576: return run(std::integral_constant<int, 36>{});  // the latent row
    case 512: return run(std::integral_constant<int, 32>{});
    case 256: return run(std::integral_constant<int, 16>{});
    case 128: return run(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
    }
}

void destroy_projection_state(sa_handle_s &h) { (void)h; }

}  // namespace sa
