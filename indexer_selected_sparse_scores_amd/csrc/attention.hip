// Softmax attention over the indexer-selected rows on gfx950.
//
// For query row r and head h: O = sum_{s in sel(r)} softmax_s(scale q_h . K_s) V_s -- the
// "execute main attention only on selected tokens" step of "Sparse Attention and RL
// Optimization: Three Technical Breakthroughs in LLM Post-Training", section 2.5, and of
// "Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and
// Verifiable Synthetic Data", section 2.4.  In decode only the selected rows of the paged
// cache are read (that page, section 2.3).
//
// attn_latent_mfma_kernel serves the latent layout in prefill (bf16, 16 heads sharing one
// 576-wide row per token whose first 512 columns are the value).  A 4-wave workgroup walks
// the selected rows of one query in chunks of 32, gathered whole with 16-byte loads (eight
// lanes per row) into LDS, the next chunk in flight while the current one is computed, so
// every 1152-byte row is read once for all 16 heads.  Logits and P.V run on v_mfma_f32_16x16x32_bf16 with
// an online softmax (running max / sum per head, exp2 with the log2(e) factor folded into
// the scale).  P enters the MFMA as a bf16 hi part plus a bf16 residual, so the weights keep
// ~16 mantissa bits.
//
// attn_decode_lds_kernel serves the latent layout in decode: the same math per chunk, with
// the selected rows of one sequence split into 512-row ranges across workgroups, each range
// staged whole rows at a time into LDS by direct global-to-LDS loads; attn_merge_kernel then
// merges the partial (max, sum, accumulator) states.
//
// attn_generic_kernel serves every other shape (fp32 or bf16): one workgroup per (row,
// head), logits in LDS, two-pass softmax.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

namespace {

__device__ __forceinline__ int64_t visible_len(const Visibility &vis, int64_t r, uint32_t *err)
{
    if (!vis.ctx_len) return vis.causal_row0 + r + 1;
    int64_t n = vis.ctx_len[r];
    if (n < 1 || n > vis.max_ctx) {
        flag_error(err, SA_DEVERR_CTX_LEN);
        return 0;
    }
    return n;
}

__device__ __forceinline__ int64_t budget(const Selection &sel, int64_t r, uint32_t *err)
{
    int64_t k = sel.k_per_row ? (int64_t)sel.k_per_row[r] : (int64_t)sel.k;
    if (k < 1 || k > sel.k) {
        flag_error(err, SA_DEVERR_TOPK);
        return 0;
    }
    return k;
}

// Element offset of token s of sequence b (the sequence of the query row, RowSource::seq_of), or
// -1 if its page is invalid.
__device__ __forceinline__ int64_t token_offset(const RowSource &src, int64_t b, int64_t s)
{
    if (!src.block_table) return s * src.row_elems;
    int32_t page = src.block_table[b * src.max_blocks + s / src.page_size];
    if (page < 0 || page >= src.n_pages) return -1;
    return ((int64_t)page * src.page_size + s % src.page_size) * src.row_elems;
}

// ---------------------------------------------------------------------------------------
// Latent layout, MFMA
// ---------------------------------------------------------------------------------------
constexpr int kLH = 16;         // query heads
constexpr int kLDqk = 576;      // key width
constexpr int kLDv = 512;       // value width (leading columns of the key row)
constexpr int kChunk = 32;      // selected rows per chunk
constexpr int kAWaves = 4;
constexpr int kAThreads = kAWaves * kWave;
constexpr int kLdsRow = kLDqk * 2 + 16;                 // padded LDS row (bytes): 292 dwords, 36 mod 64 banks
constexpr int kKSteps = kLDqk / 32;                     // 18 k-steps of the logits MFMA
constexpr int kKHalf = kKSteps / 2;                     // each wave pair takes half of them
constexpr int kLogitLd = kChunk + 4;                    // padded per-head row of logits (floats)
constexpr int kColsPerWave = kLDv / kAWaves;            // 128 value columns per wave
constexpr int kNTiles = kColsPerWave / 16;              // 8 MFMA column tiles per wave
constexpr int kHeadsPerWave = kLH / kAWaves;            // softmax heads owned by a wave (4)

struct AttnShared {
    unsigned char rows[kChunk * kLdsRow];   // the current chunk's selected rows (all 576 columns)
    float logits[2][kLH * kLogitLd];        // partial logits of the two K-halves, [head][slot]
    uint4 p_hi[kLH][4];                     // P as the A operand of P.V: [head][lane group]
    uint4 p_lo[kLH][4];                     //   (8 bf16 each), hi part and bf16 residual
    float alpha[kLH];                       // per-head rescale of this chunk
    float inv_l[kLH];                       // per-head 1 / softmax sum (end of the row)
    int64_t row_off[2][kChunk];             // element offsets of a chunk's rows (-1: none)
};

// Element offset of selected slot j of a query row of sequence tb, -1 if the slot is unused or
// invalid.
__device__ __forceinline__ int64_t slot_offset(const RowSource &kv, const int32_t *idx_row, int64_t tb,
                                               int64_t j, int64_t j_end, int64_t visible, uint32_t *err)
{
    if (j >= j_end) return -1;
    const int64_t s = idx_row[j];
    if (s >= visible) flag_error(err, SA_DEVERR_INDEX_RANGE);
    if (s < 0 || s >= visible) return -1;
    const int64_t off = token_offset(kv, tb, s);
    if (off < 0) flag_error(err, SA_DEVERR_BLOCK_TABLE);
    return off;
}

// The P.V contraction runs over the 32 rows of a chunk in an order of our choosing, as long
// as P and V agree.  MFMA k index 8 g + j (lane group g = lane / 16, j = 0..7) is row 8 g + 2 j
// (j < 4) or 8 g + 2 (j - 4) + 1 (j >= 4): the V fragment is then two transposing LDS reads
// over rows two apart, which fall in disjoint banks.  slot_of_row inverts the map; logits are
// stored at their slot so that P is produced in k order.
__device__ __forceinline__ int slot_of_row(int row)
{
    const int w = row & 7;
    return (row & ~7) | ((w & 1) << 2) | (w >> 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Lane l of each 16-lane group gets column c0 + l % 16 of the 4 rows whose 8-byte pieces the
// group's lanes point at (ds_read_b64_tr_b16: lane i, element e comes from element i % 4 of
// the row addressed by lane 4 e + i / 4).
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(reinterpret_cast<uintptr_t>(p)));
}

// Max / sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp_mov<kDppXor1>(x));
    x = fmaxf(x, dpp_mov<kDppXor2>(x));
    x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
    return fmaxf(x, dpp_mov<kDppRowMirror>(x));
}
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    x += dpp_mov<kDppRowHalfMirror>(x);
    return x + dpp_mov<kDppRowMirror>(x);
}

// One 4-wave workgroup = one query row (all 16 heads) and a range of its selected rows, in
// chunks of 32 rows; three workgroups share a compute unit, so one's barriers and memory
// waits overlap the others' work.  The selected rows are gathered whole (eight lanes per row,
// 128-byte lines), one chunk in flight in registers while the previous one sits in LDS: a
// gather of whole lines moves more bytes per second through the fabric than one in which each
// lane fetches only the pieces its own MFMAs use.  Per chunk:
//  * logits: wave w takes rows 16 (w % 2) .. +15 over half w / 2 of the 576-wide contraction
//    (v_mfma_f32_16x16x32_bf16, q fragments in registers, K fragments from LDS).
//  * online softmax: wave w owns heads 4w .. 4w+3 (running max / sum, exp2 with log2(e)
//    folded into the scale) and publishes P as bf16 hi + residual (~16 mantissa bits).
//  * P.V: every wave accumulates 128 of the 512 value columns, with V fragments from
//    transposing LDS reads.
// Row offsets run two chunks ahead (index load, then page lookup, then use).
__global__ __launch_bounds__(kAThreads, 3) void attn_latent_mfma_kernel(
    const uint16_t *__restrict__ q, int64_t n_rows, RowSource kv, Visibility vis, Selection sel,
    float scale_log2, float *__restrict__ out, float *__restrict__ lse, uint32_t *err)
{
    __shared__ __attribute__((aligned(16))) AttnShared sh;

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int hh = lane % 16, grp = lane / 16;
    const int64_t r = blockIdx.x;
    uint32_t *err0 = tid == 0 ? err : nullptr;
    const int64_t visible = visible_len(vis, r, err0);
    const int64_t kr = budget(sel, r, err0);
    const int64_t m = kr < visible ? kr : visible;
    const int64_t j_begin = 0, j_end = m;
    const int64_t tb = kv.block_table ? kv.seq_of(r) : r;  // block-table row of the sequence
    const int32_t *idx_row = sel.idx + r * sel.idx_ld;
    const uint16_t *kv_base = reinterpret_cast<const uint16_t *>(kv.base);
    const int n_chunks = (int)((j_end - j_begin + kChunk - 1) / kChunk);

    const int nt_qk = wave & 1, kh = wave >> 1;
    const int my_row = 16 * nt_qk + hh;  // the chunk row whose logits this lane's MFMA B fragments cover
    bf16x8 qa[kKHalf];
    const uint16_t *qr = q + (r * kLH + hh) * kLDqk;
#pragma unroll
    for (int i = 0; i < kKHalf; ++i) qa[i] = as_bf16x8(load16(qr + 32 * (kKHalf * kh + i) + 8 * grp));

    // offsets of chunks 0 and 1; the index of chunk 2 waits in a register
    int64_t pend_j = j_begin + 2 * kChunk + tid;  // slot whose index `pend_s` holds
    // 32-bit as loaded: widened only where it is used, a chunk later (widening it at the load
    // would make the wave wait for the load right there)
    int32_t pend_s = -1;
    if (tid < kChunk) {
        sh.row_off[0][tid] = slot_offset(kv, idx_row, tb, j_begin + tid, j_end, visible, err);
        sh.row_off[1][tid] = slot_offset(kv, idx_row, tb, j_begin + kChunk + tid, j_end, visible, err);
        if (pend_j < j_end) pend_s = idx_row[pend_j];
    }
    __syncthreads();

    // Gather: eight lanes per selected row, wave w taking rows 8 w .. 8 w + 7 of a chunk; lane l copies
    // the 16-byte pieces l % 8 + 8 i (i = 0..8) of row 8 w + l / 8, so each load instruction reads whole
    // 128-byte lines of 8 rows.  An unused slot reads the first row of the source and is zeroed (no
    // branch around the loads).
    const int g_row = 8 * wave + lane / 8, g_col = lane % 8;
    uint4 g[kKHalf];
    auto gather = [&](int buf) {
        const int64_t off = sh.row_off[buf][g_row];
        const uint16_t *src = kv_base + (off >= 0 ? off : 0) + 8 * g_col;
#pragma unroll
        for (int i = 0; i < kKHalf; ++i) g[i] = load16(src + 64 * i);
        if (off < 0) {
#pragma unroll
            for (int i = 0; i < kKHalf; ++i) g[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < kKHalf; ++i)
            *reinterpret_cast<uint4 *>(sh.rows + g_row * kLdsRow + 16 * (g_col + 8 * i)) = g[i];
    };
    gather(0);
    stash();
    gather(1);
    __syncthreads();

    const float neg_inf = -__builtin_inff();
    // softmax state of head 4 wave + lane / 16 (log2 domain), owned by this wave
    const int sm_head = kHeadsPerWave * wave + grp;
    float m_run = neg_inf, l_run = 0.f;
    f32x4 acc[kNTiles];  // O[4 grp + i][128 wave + 16 nt + hh]
#pragma unroll
    for (int nt = 0; nt < kNTiles; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
    for (int c = 0; c < n_chunks; ++c) {
        // rows = chunk c, g = chunk c + 1 in flight, row_off[c & 1] = chunk c,
        // row_off[(c + 1) & 1] = chunk c + 1
        // Slot pend_j (chunk c + 2): its index arrived during the previous chunk; its page
        // lookup and the index of chunk c + 3 are issued before this chunk's gather loads, so
        // the memory counter reaches them first, and they are consumed after the compute.
        int64_t off_next = -1;
        int32_t page = 0;
        bool page_pending = false;
        if (tid < kChunk && pend_j < j_end) {
            const int64_t ps = pend_s;
            if (ps >= visible) flag_error(err, SA_DEVERR_INDEX_RANGE);
            if (ps >= 0 && ps < visible) {
                if (kv.block_table) {
                    page = kv.block_table[tb * kv.max_blocks + ps / kv.page_size];
                    page_pending = true;
                } else {
                    off_next = ps * kv.row_elems;
                }
            }
        }
        const int64_t s_next = pend_s;
        pend_j += kChunk;
        pend_s = -1;
        if (tid < kChunk && pend_j < j_end) pend_s = idx_row[pend_j];

        // partial logits of rows 16 nt_qk + (0..15), heads 0..15, k-steps of half kh; lane (hh, grp)
        // reads its B fragments (row my_row, dims 32 (9 kh + i) + 8 grp .. +7) from the chunk in LDS
        {
            const unsigned char *kb = sh.rows + my_row * kLdsRow + 2 * (32 * kKHalf * kh + 8 * grp);
            uint4 kf[kKHalf];
#pragma unroll
            for (int i = 0; i < kKHalf; ++i) kf[i] = *reinterpret_cast<const uint4 *>(kb + 64 * i);
            f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = {0.f, 0.f, 0.f, 0.f};  // two chains
#pragma unroll
            for (int i = 0; i < kKHalf; i += 2) {
                sa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i], as_bf16x8(kf[i]), sa0, 0, 0, 0);
                if (i + 1 < kKHalf)
                    sa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i + 1], as_bf16x8(kf[i + 1]), sa1, 0, 0, 0);
            }
            const f32x4 sacc = sa0 + sa1;
            // output (head 4 grp + i, row my_row)
            const bool valid = sh.row_off[c & 1][my_row] >= 0;
            const int slot = slot_of_row(my_row);
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.logits[kh][(4 * grp + i) * kLogitLd + slot] = valid ? sacc[i] : neg_inf;
        }
        __syncthreads();

        // online softmax of head sm_head over the 32 slots: this lane takes slots l % 16 and
        // 16 + l % 16
        {
            const int sl = hh;
            const float *lg0 = &sh.logits[0][sm_head * kLogitLd];
            const float *lg1 = &sh.logits[1][sm_head * kLogitLd];
            const float x0 = (lg0[sl] + lg1[sl]) * scale_log2;
            const float x1 = (lg0[16 + sl] + lg1[16 + sl]) * scale_log2;
            const float cmax = row16_max(fmaxf(x0, x1));
            const float m_new = fmaxf(m_run, cmax);
            const bool any = m_new != neg_inf;
            const float alpha = any ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            const float p0 = any ? __builtin_amdgcn_exp2f(x0 - m_new) : 0.f;
            const float p1 = any ? __builtin_amdgcn_exp2f(x1 - m_new) : 0.f;
            const float psum = row16_sum(p0 + p1);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            // slot s is MFMA k index s (lane group s / 8, element s % 8)
            const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
            const __bf16 r0 = (__bf16)(p0 - (float)h0), r1 = (__bf16)(p1 - (float)h1);
            __bf16 *ph = reinterpret_cast<__bf16 *>(&sh.p_hi[sm_head][0]);
            __bf16 *pl = reinterpret_cast<__bf16 *>(&sh.p_lo[sm_head][0]);
            ph[sl] = h0;
            pl[sl] = r0;
            ph[16 + sl] = h1;
            pl[16 + sl] = r1;
            if (sl == 0) sh.alpha[sm_head] = alpha;
        }
        __syncthreads();

        // rescale the accumulator rows (heads 4 grp + i), then P.V over the 32 rows
        {
            const float4 al = *reinterpret_cast<const float4 *>(&sh.alpha[4 * grp]);
#pragma unroll
            for (int nt = 0; nt < kNTiles; ++nt) {
                acc[nt][0] *= al.x;
                acc[nt][1] *= al.y;
                acc[nt][2] *= al.z;
                acc[nt][3] *= al.w;
            }
        }
        // B fragment of lane (hh, grp): rows 8 grp + {0, 2, 4, 6} then {1, 3, 5, 7}, column
        // 128 wave + 16 nt + hh, via two transposing reads whose lanes point at row
        // 8 grp + 2 (hh / 4) (+1) and columns 128 wave + 16 nt + 4 (hh % 4) .. +3.
        {
            const bf16x8 pa_hi = as_bf16x8(sh.p_hi[hh][grp]);
            const bf16x8 pa_lo = as_bf16x8(sh.p_lo[hh][grp]);
            const unsigned char *vb0 = sh.rows + (8 * grp + 2 * (hh / 4)) * kLdsRow +
                                       2 * (kColsPerWave * wave + 4 * (hh % 4));
#pragma unroll
            for (int nt = 0; nt < kNTiles; ++nt) {
                const unsigned char *vb = vb0 + 2 * 16 * nt;
                const s16x4 lo4 = lds_read_tr16(vb);
                const s16x4 hi4 = lds_read_tr16(vb + kLdsRow);
                const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, b, acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b, acc[nt], 0, 0, 0);
            }
        }
        // row_off[c & 1] was last read by this chunk's logits (before the barriers above); it
        // now takes chunk c + 2, which the gather after the barrier below reads.
        // The page lookup is consumed here on every path, so no wait for it is left pending
        // into the next chunk (where `page` is reset).
        asm volatile("" : : "v"(page));
        if (page_pending) {
            if (page >= 0 && page < kv.n_pages) {
                off_next = ((int64_t)page * kv.page_size + s_next % kv.page_size) * kv.row_elems;
            } else {
                flag_error(err, SA_DEVERR_BLOCK_TABLE);
            }
        }
        if (tid < kChunk) sh.row_off[c & 1][tid] = off_next;
        __syncthreads();  // every wave is done with rows, logits and P; row_off is published
        // chunk c + 1 into LDS and chunk c + 2 in flight, both unconditional: past the last chunk
        // they store values nothing reads and load the source's first row (offsets -1).  Issued at raised
        // wave priority, so that the loads leave ahead of the other workgroups' softmax and MFMA work.
        __builtin_amdgcn_s_setprio(1);
        stash();
        gather(c & 1);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    }

    if (hh == 0) sh.inv_l[sm_head] = l_run > 0.f ? 1.f / l_run : 0.f;
    if (lse && hh == 0) lse[r * kLH + sm_head] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : neg_inf;
    __syncthreads();
    const float4 iv = *reinterpret_cast<const float4 *>(&sh.inv_l[4 * grp]);
    const float ivs[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float *orow = out + (r * kLH + 4 * grp + i) * kLDv + kColsPerWave * wave + hh;
#pragma unroll
        for (int nt = 0; nt < kNTiles; ++nt) orow[16 * nt] = acc[nt][i] * ivs[i];
    }
}

// ---------------------------------------------------------------------------------------
// Latent layout, decode: selected rows staged in LDS by direct loads
// ---------------------------------------------------------------------------------------
constexpr int kDSplitRows = 512;                  // selected rows per decode workgroup (many rows: 1024)
constexpr int kDSplitRowsMax = 2 * kDSplitRows;
constexpr int kRing = 3;                          // chunk slots in LDS: two chunks in flight
constexpr int kRowBytes = kLDqk * 2;              // 1152
constexpr int kSlotBytes = kChunk * kRowBytes;    // 36864
constexpr int kBlkBytes = 8 * kRowBytes;          // rows 8w .. 8w + 7 of a chunk
constexpr int kSegs = kRowBytes / 128;            // direct loads per wave per chunk
constexpr size_t kRingBytes = (size_t)kRing * kSlotBytes;

__device__ __attribute__((aligned(16))) uint16_t g_zero_row[kLDqk];  // source of unused slots (zeros)

// Byte offset of byte b of row R of a chunk in its LDS slot.  Rows 8w .. 8w + 7 form block w;
// bytes 128 s .. 128 s + 127 of the block's rows form its 1 KB segment s, inside which row r = R % 8
// keeps its 16-byte piece p at position 8 (r ^ (w & 1)) + (p ^ r).  One direct load (64 lanes x
// 16 bytes, written lane after lane) fills one segment from 128 contiguous bytes of each of 8 rows;
// the swizzle spreads the operand reads below (one piece of 16 rows from two blocks, or 8-byte
// pieces of 8 rows) over distinct LDS banks.
__device__ __forceinline__ uint32_t slot_byte(int R, int b)
{
    const int w = R >> 3, r = R & 7, p = b >> 4;
    return (uint32_t)(kBlkBytes * w + 1024 * (p >> 3) + 16 * (8 * (r ^ (w & 1)) + ((p & 7) ^ r)) + (b & 15));
}

// Workgroup barrier ordering LDS accesses only: __syncthreads would also wait for every direct load
// in flight (its fence waits for the whole memory counter).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt for the memory counter only (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int kVm>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((kVm & 0xF) | ((kVm >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Decode attention over one sequence's selected rows, split in ranges of 512 (or, for many rows, 1024)
// across workgroups (partials merged by attn_merge_kernel).  The rows of a 32-row chunk reach LDS through direct
// global-to-LDS loads, 128 contiguous bytes of a row per lane octet, two chunks ahead of the one
// being computed, so no register holds a row in flight and every row is read once at the full
// gather rate.  Per chunk the math is that of attn_latent_mfma_kernel: logits on
// v_mfma_f32_16x16x32_bf16 with K read from LDS, online softmax per head, P.V with V fragments from
// transposing LDS reads.  The ring is read only through inline asm: the compiler cannot tell which
// slot an in-flight direct load writes, and would otherwise wait for all of them before every read.
__global__ __launch_bounds__(kAThreads, 1) void attn_decode_lds_kernel(
    const uint16_t *__restrict__ q, RowSource kv, Visibility vis, Selection sel, float scale_log2,
    int split_rows, int n_splits, float *__restrict__ part_o, float *__restrict__ part_ml, uint32_t *err)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char ring[];  // kRing slots of kSlotBytes
    __shared__ int64_t rows[kDSplitRowsMax];  // pool row of each selected slot of the range (-1: none)
    __shared__ float logits[2][kLH * kLogitLd];
    __shared__ uint4 p_hi[kLH][4], p_lo[kLH][4];
    __shared__ float alpha_s[kLH];

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int hh = lane % 16, grp = lane / 16;
    // row rotated by the range: workgroups reach the XCDs round-robin by linear id, so with a row count that
    // is a multiple of 8 every range of row r would run on XCD r % 8, and rows' unequal budgets would load the
    // XCDs unequally; rotated, the ranges of a row spread over the XCDs
    const int split = (int)blockIdx.y;
    const int64_t r = ((int64_t)blockIdx.x + split) % gridDim.x;
    uint32_t *err0 = (tid == 0 && split == 0) ? err : nullptr;
    const int64_t visible = visible_len(vis, r, err0);
    const int64_t kr = budget(sel, r, err0);
    const int64_t m = kr < visible ? kr : visible;
    const int64_t j_begin = (int64_t)split * split_rows;
    if (j_begin >= m) return;  // the merge kernel ignores unused splits
    const int64_t tb = kv.block_table ? kv.seq_of(r) : r;  // block-table row of the sequence
    const int n_here = (int)(m - j_begin < split_rows ? m - j_begin : split_rows);
    const int n_chunks = (n_here + kChunk - 1) / kChunk;
    const int32_t *idx_row = sel.idx + r * sel.idx_ld + j_begin;

    const int nt_qk = wave & 1, kh = wave >> 1;
    bf16x8 qa[kKHalf];
    const uint16_t *qr = q + (r * kLH + hh) * kLDqk;
#pragma unroll
    for (int i = 0; i < kKHalf; ++i) qa[i] = as_bf16x8(load16(qr + 32 * (kKHalf * kh + i) + 8 * grp));

    // pool row of every selected slot of the range: all indices, then all page lookups
    {
        // split_rows is 512 or 1024: the second half of the loops runs only for 1024-row ranges
        int32_t sv[kDSplitRowsMax / kAThreads];
#pragma unroll
        for (int k = 0; k < kDSplitRowsMax / kAThreads; ++k) {
            const int j = tid + kAThreads * k;
            sv[k] = j < n_here ? idx_row[j] : -1;
        }
#pragma unroll
        for (int k = 0; k < kDSplitRowsMax / kAThreads; ++k) {
            const int j = tid + kAThreads * k;
            if (kAThreads * k >= split_rows) break;
            const int64_t s = sv[k];
            int64_t row = -1;
            if (j < n_here) {
                if (s >= visible) flag_error(err, SA_DEVERR_INDEX_RANGE);
                if (s >= 0 && s < visible) {
                    if (kv.block_table) {
                        const int32_t page = kv.block_table[tb * kv.max_blocks + s / kv.page_size];
                        if (page >= 0 && page < kv.n_pages)
                            row = (int64_t)page * kv.page_size + s % kv.page_size;
                        else
                            flag_error(err, SA_DEVERR_BLOCK_TABLE);
                    } else {
                        row = s;
                    }
                }
            }
            rows[j] = row;
        }
    }
    __syncthreads();

    // direct loads of chunk c into slot c % kRing: lane l of wave w copies, of chunk row 8w + dr,
    // the pieces dp, dp + 8, ..., dp + 64 (one 128-byte segment per load); unused slots copy zeros
    const int dr = (lane >> 3) ^ (wave & 1), dp = (lane & 7) ^ dr;
    const unsigned char *kv_bytes = reinterpret_cast<const unsigned char *>(kv.base);
    auto issue = [&](int c) {
        const int jr = kChunk * c + 8 * wave + dr;
        const int64_t row = jr < n_here ? rows[jr] : -1;
        const unsigned char *src = (row >= 0 ? kv_bytes + row * kRowBytes
                                             : reinterpret_cast<const unsigned char *>(g_zero_row)) + 16 * dp;
        unsigned char *dst = ring + (c % kRing) * kSlotBytes + kBlkBytes * wave;
#pragma unroll
        for (int i = 0; i < kSegs; ++i)
            __builtin_amdgcn_global_load_lds(src + 128 * i, (__attribute__((address_space(3))) void *)(dst + 1024 * i),
                                             16, 0, 0);
    };

    // this lane's operand offsets within a slot: K pieces of the logits MFMAs (row 16 nt_qk + hh,
    // piece 4 (9 kh + i) + grp) and the 8-byte V pieces of the P.V fragments (rows 8 grp + 2 (hh / 4)
    // and +1, columns 128 wave + 16 nt + 4 (hh % 4) .. +3)
    uint32_t koff[kKHalf], voff[kNTiles][2];
#pragma unroll
    for (int i = 0; i < kKHalf; ++i) koff[i] = slot_byte(16 * nt_qk + hh, 16 * (4 * (kKHalf * kh + i) + grp));
#pragma unroll
    for (int nt = 0; nt < kNTiles; ++nt) {
        const int col = kColsPerWave * wave + 16 * nt + 4 * (hh % 4);
        voff[nt][0] = slot_byte(8 * grp + 2 * (hh / 4), 2 * col);
        voff[nt][1] = slot_byte(8 * grp + 2 * (hh / 4) + 1, 2 * col);
    }
    const uint32_t ring_lds = (uint32_t)reinterpret_cast<uintptr_t>(ring);

    const float neg_inf = -__builtin_inff();
    const int sm_head = kHeadsPerWave * wave + grp;  // softmax state owned by this lane group
    float m_run = neg_inf, l_run = 0.f;
    f32x4 acc[kNTiles];  // O[4 grp + i][128 wave + 16 nt + hh]
#pragma unroll
    for (int nt = 0; nt < kNTiles; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int c = 0; c < kRing - 1; ++c)
        if (c < n_chunks) issue(c);
#pragma unroll 1
    for (int c = 0; c < n_chunks; ++c) {
        // this wave's loads of chunk c are done once only the later chunks' are outstanding (no other
        // memory instruction is issued in the loop); the barrier makes every wave's part visible and
        // closes the previous chunk, whose slot takes chunk c + kRing - 1
        static_assert(kRing >= 2 && kRing <= 4, "waits below");
        const int later = n_chunks - 1 - c < kRing - 2 ? n_chunks - 1 - c : kRing - 2;  // chunks issued after c
        if (later >= 2)
            wait_vmcnt<2 * kSegs>();
        else if (later == 1)
            wait_vmcnt<kSegs>();
        else
            wait_vmcnt<0>();
        lds_barrier();
        if (c + kRing - 1 < n_chunks) issue(c + kRing - 1);
        const uint32_t sb = ring_lds + (uint32_t)((c % kRing) * kSlotBytes);

        // partial logits of rows 16 nt_qk + (0..15), heads 0..15, k-steps of half kh
        {
            bf16x8 kf[kKHalf];
#pragma unroll
            for (int i = 0; i < kKHalf; ++i) asm volatile("ds_read_b128 %0, %1" : "=v"(kf[i]) : "v"(sb + koff[i]));
            // the wait is tied to the loaded registers, so nothing that reads them moves above it
            static_assert(kKHalf == 9, "one operand per piece below");
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(kf[0]), "+v"(kf[1]), "+v"(kf[2]), "+v"(kf[3]), "+v"(kf[4]), "+v"(kf[5]), "+v"(kf[6]),
                           "+v"(kf[7]), "+v"(kf[8])
                         :
                         : "memory");
            f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = {0.f, 0.f, 0.f, 0.f};  // two chains
#pragma unroll
            for (int i = 0; i < kKHalf; i += 2) {
                sa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i], kf[i], sa0, 0, 0, 0);
                if (i + 1 < kKHalf) sa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i + 1], kf[i + 1], sa1, 0, 0, 0);
            }
            const f32x4 sacc = sa0 + sa1;
            const int my_row = 16 * nt_qk + hh;
            const int jr = kChunk * c + my_row;
            const bool valid = jr < n_here && rows[jr] >= 0;
            const int slot = slot_of_row(my_row);
#pragma unroll
            for (int i = 0; i < 4; ++i) logits[kh][(4 * grp + i) * kLogitLd + slot] = valid ? sacc[i] : neg_inf;
        }
        lds_barrier();

        // online softmax of head sm_head over the 32 slots (this lane: slots l % 16 and 16 + l % 16)
        {
            const int sl = hh;
            const float *lg0 = &logits[0][sm_head * kLogitLd];
            const float *lg1 = &logits[1][sm_head * kLogitLd];
            const float x0 = (lg0[sl] + lg1[sl]) * scale_log2;
            const float x1 = (lg0[16 + sl] + lg1[16 + sl]) * scale_log2;
            const float cmax = row16_max(fmaxf(x0, x1));
            const float m_new = fmaxf(m_run, cmax);
            const bool any = m_new != neg_inf;
            const float alpha = any ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            const float p0 = any ? __builtin_amdgcn_exp2f(x0 - m_new) : 0.f;
            const float p1 = any ? __builtin_amdgcn_exp2f(x1 - m_new) : 0.f;
            const float psum = row16_sum(p0 + p1);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
            const __bf16 r0 = (__bf16)(p0 - (float)h0), r1 = (__bf16)(p1 - (float)h1);
            __bf16 *ph = reinterpret_cast<__bf16 *>(&p_hi[sm_head][0]);
            __bf16 *pl = reinterpret_cast<__bf16 *>(&p_lo[sm_head][0]);
            ph[sl] = h0;
            pl[sl] = r0;
            ph[16 + sl] = h1;
            pl[16 + sl] = r1;
            if (sl == 0) alpha_s[sm_head] = alpha;
        }
        lds_barrier();

        // rescale the accumulator rows (heads 4 grp + i), then P.V over the 32 rows
        {
            const float4 al = *reinterpret_cast<const float4 *>(&alpha_s[4 * grp]);
#pragma unroll
            for (int nt = 0; nt < kNTiles; ++nt) {
                acc[nt][0] *= al.x;
                acc[nt][1] *= al.y;
                acc[nt][2] *= al.z;
                acc[nt][3] *= al.w;
            }
            const bf16x8 pa_hi = as_bf16x8(p_hi[hh][grp]);
            const bf16x8 pa_lo = as_bf16x8(p_lo[hh][grp]);
            s16x4 vlo[kNTiles], vhi[kNTiles];
#pragma unroll
            for (int nt = 0; nt < kNTiles; ++nt) {
                asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vlo[nt]) : "v"(sb + voff[nt][0]));
                asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vhi[nt]) : "v"(sb + voff[nt][1]));
            }
            static_assert(kNTiles == 8, "one operand per fragment below");
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(vlo[0]), "+v"(vlo[1]), "+v"(vlo[2]), "+v"(vlo[3]), "+v"(vlo[4]), "+v"(vlo[5]),
                           "+v"(vlo[6]), "+v"(vlo[7]), "+v"(vhi[0]), "+v"(vhi[1]), "+v"(vhi[2]), "+v"(vhi[3]),
                           "+v"(vhi[4]), "+v"(vhi[5]), "+v"(vhi[6]), "+v"(vhi[7])
                         :
                         : "memory");
#pragma unroll
            for (int nt = 0; nt < kNTiles; ++nt) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[nt], vhi[nt], 0, 1, 2, 3, 4, 5, 6, 7));
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, b, acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b, acc[nt], 0, 0, 0);
            }
        }
    }

    const int64_t slot = r * n_splits + split;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float *prow = part_o + (slot * kLH + 4 * grp + i) * kLDv + kColsPerWave * wave + hh;
#pragma unroll
        for (int nt = 0; nt < kNTiles; ++nt) prow[16 * nt] = acc[nt][i];
    }
    if (hh == 0) {
        part_ml[(slot * kLH + sm_head) * 2 + 0] = m_run;
        part_ml[(slot * kLH + sm_head) * 2 + 1] = l_run;
    }
}

// Merge the per-split softmax states of each decode row: O = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s with M = max_s m_s.  One 128-thread workgroup per (row, head), four
// value columns per thread.  Every split's (m, l) and o are loaded in one batch (at most
// kMergeMaxSplits: top-k <= 8192 in ranges of >= 512), then summed in split order.
constexpr int kMergeMaxSplits = 16;
__global__ __launch_bounds__(128) void attn_merge_kernel(
    Visibility vis, Selection sel, int split_rows, int n_splits, const float *__restrict__ part_o,
    const float *__restrict__ part_ml, float *__restrict__ out, float *__restrict__ lse)
{
    const int64_t r = blockIdx.x / kLH;
    const int h = blockIdx.x % kLH;
    int64_t visible = vis.ctx_len ? (int64_t)vis.ctx_len[r] : vis.causal_row0 + r + 1;
    if (vis.ctx_len && (visible < 1 || visible > vis.max_ctx)) visible = 0;
    int64_t k = sel.k_per_row ? (int64_t)sel.k_per_row[r] : (int64_t)sel.k;
    if (k < 1 || k > sel.k) k = 0;
    const int64_t m = k < visible ? k : visible;
    const int used = (int)((m + split_rows - 1) / split_rows);
    const float neg_inf = -__builtin_inff();
    float ms[kMergeMaxSplits], ls[kMergeMaxSplits];
    float4 o[kMergeMaxSplits];
#pragma unroll
    for (int s = 0; s < kMergeMaxSplits; ++s) {
        if (s < used) {
            const int64_t slot = (r * n_splits + s) * kLH + h;
            const float2 ml = reinterpret_cast<const float2 *>(part_ml)[slot];
            ms[s] = ml.x;
            ls[s] = ml.y;
            o[s] = reinterpret_cast<const float4 *>(part_o + slot * kLDv)[threadIdx.x];
        }
    }
    float M = neg_inf;
#pragma unroll
    for (int s = 0; s < kMergeMaxSplits; ++s)
        if (s < used) M = fmaxf(M, ms[s]);
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    if (M != neg_inf) {
#pragma unroll
        for (int s = 0; s < kMergeMaxSplits; ++s) {
            if (s < used && ms[s] != neg_inf) {  // a split without a visible row adds nothing
                const float f = exp2f(ms[s] - M);
                den = fmaf(ls[s], f, den);
                num.x = fmaf(o[s].x, f, num.x);
                num.y = fmaf(o[s].y, f, num.y);
                num.z = fmaf(o[s].z, f, num.z);
                num.w = fmaf(o[s].w, f, num.w);
            }
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    reinterpret_cast<float4 *>(out + (r * kLH + h) * (int64_t)kLDv)[threadIdx.x] =
        make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
    if (lse && threadIdx.x == 0) lse[r * kLH + h] = den > 0.f ? (M + __log2f(den)) * kLn2 : neg_inf;
}

// ---------------------------------------------------------------------------------------
// Generic shapes (VALU)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float v, float *tmp, bool is_max)
{
    const int lane = lane_id(), wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        float u = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, u) : v + u;
    }
    if (lane == 0) tmp[wave] = v;
    __syncthreads();
    float r = tmp[0];
    for (int i = 1; i < nw; ++i) r = is_max ? fmaxf(r, tmp[i]) : r + tmp[i];
    __syncthreads();
    return r;
}

template <class T>
__global__ __launch_bounds__(256) void attn_generic_kernel(
    const T *__restrict__ q, int H, int H_kv, int d_qk, int d_v, RowSource kv, RowSource vsrc,
    Visibility vis, Selection sel, float scale_log2, float *__restrict__ out,
    float *__restrict__ lse, uint32_t *err)
{
    extern __shared__ float smem[];
    __shared__ float red[4];
    float *qh = smem;                 // [d_qk]
    float *pw = smem + d_qk;          // [k]: logits, then softmax weights
    const int64_t r = blockIdx.x;
    const int h = blockIdx.y;
    const int g = (int)((int64_t)h * H_kv / H);
    uint32_t *err0 = (threadIdx.x == 0 && h == 0) ? err : nullptr;
    const int64_t visible = visible_len(vis, r, err0);
    const int64_t kr = budget(sel, r, err0);
    const int64_t m = kr < visible ? kr : visible;
    const int32_t *idx_row = sel.idx + r * sel.idx_ld;
    const T *kbase = reinterpret_cast<const T *>(kv.base);
    const T *vbase = reinterpret_cast<const T *>(vsrc.base);
    const int64_t tb = kv.block_table ? kv.seq_of(r) : r;  // block-table row of the sequence
    for (int c = threadIdx.x; c < d_qk; c += blockDim.x) qh[c] = load_elem(q + (r * H + h) * (int64_t)d_qk + c);
    __syncthreads();

    const float neg_inf = -__builtin_inff();
    float mx = neg_inf;
    for (int64_t j = threadIdx.x; j < m; j += blockDim.x) {
        const int64_t s = idx_row[j];
        float l = neg_inf;
        if (s >= visible && h == 0) flag_error(err, SA_DEVERR_INDEX_RANGE);
        if (s >= 0 && s < visible) {
            const int64_t off = token_offset(kv, tb, s);
            if (off >= 0) {
                const T *kr_ = kbase + off + (int64_t)g * d_qk;
                float dot = 0.f;
                for (int c = 0; c < d_qk; ++c) dot = fmaf(qh[c], load_elem(kr_ + c), dot);
                l = dot * scale_log2;
            } else if (h == 0) {
                flag_error(err, SA_DEVERR_BLOCK_TABLE);
            }
        }
        pw[j] = l;
        mx = fmaxf(mx, l);
    }
    mx = block_reduce(mx, red, true);
    float sum = 0.f;
    for (int64_t j = threadIdx.x; j < m; j += blockDim.x) {
        const float p = mx == neg_inf ? 0.f : exp2f(pw[j] - mx);
        pw[j] = p;
        sum += p;
    }
    sum = block_reduce(sum, red, false);  // also orders the pw writes before the reads below
    for (int d = threadIdx.x; d < d_v; d += blockDim.x) {
        float a = 0.f;
        for (int64_t j = 0; j < m; ++j) {
            const float p = pw[j];
            if (p == 0.f) continue;
            const int64_t s = idx_row[j];
            const int64_t off = token_offset(vbase ? vsrc : kv, tb, s);
            const T *vr = vbase ? vbase + off + (int64_t)g * d_v : kbase + off + (int64_t)g * d_qk;
            a = fmaf(p, load_elem(vr + d), a);
        }
        out[(r * H + h) * (int64_t)d_v + d] = sum > 0.f ? a / sum : 0.f;
    }
    if (lse && threadIdx.x == 0) lse[r * H + h] = sum > 0.f ? (mx + __log2f(sum)) * kLn2 : neg_inf;
}

}  // namespace

size_t attention_workspace(const sa_handle_s &h, int64_t n_rows, bool decode)
{
    if (!decode || !h.fast_attn) return 0;
    const int64_t n_splits = (h.cfg.max_topk + kDSplitRows - 1) / kDSplitRows;
    return (size_t)n_rows * n_splits * kLH * (kLDv + 2) * sizeof(float);
}

hipError_t launch_attention(sa_handle_s &h, const void *q, int64_t n_rows, RowSource kv,
                            RowSource v, Visibility vis, Selection sel, float *out, float *lse,
                            void *ws, hipStream_t st, bool allow_split)
{
    if (n_rows <= 0) return hipSuccess;
    const float scale_log2 = h.scale * kLog2e;
    const bool decode = vis.ctx_len != nullptr && allow_split;
    if (h.fast_attn) {
        const uint16_t *qq = reinterpret_cast<const uint16_t *>(q);
        if (!decode) {
            KernelTimer timer(h, SA_KERNEL_ATTENTION, st);
            hipLaunchKernelGGL(attn_latent_mfma_kernel, dim3((unsigned)n_rows), dim3(kAThreads), 0, st, qq, n_rows,
                               kv, vis, sel, scale_log2, out, lse, h.d_err);
            return hipGetLastError();
        }
        // decode: the selected rows staged in LDS by direct loads, one range of rows per workgroup, then the merge;
        // 512-row ranges while the rows' ranges fill at most two rounds of workgroups on the CUs; beyond,
        // 1024-row ranges halve the per-workgroup start (the index and page lookups before the first chunk)
        const int64_t ranges512 = n_rows * ((h.cfg.max_topk + kDSplitRows - 1) / kDSplitRows);
        const int split_rows = ranges512 <= 2 * (int64_t)h.n_cu ? kDSplitRows : kDSplitRowsMax;
        const int n_splits = (h.cfg.max_topk + split_rows - 1) / split_rows;
        if (n_splits > kMergeMaxSplits) return hipErrorInvalidValue;  // max_topk <= 8192 keeps it <= 16
        float *part_o = reinterpret_cast<float *>(ws);
        float *part_ml = part_o + (size_t)n_rows * n_splits * kLH * kLDv;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_decode_lds_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRingBytes);
        if (e != hipSuccess) return e;
        {
            KernelTimer timer(h, SA_KERNEL_ATTENTION, st);
            hipLaunchKernelGGL(attn_decode_lds_kernel, dim3((unsigned)n_rows, (unsigned)n_splits), dim3(kAThreads),
                               kRingBytes, st, qq, kv, vis, sel, scale_log2, split_rows, n_splits, part_o, part_ml,
                               h.d_err);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        KernelTimer timer(h, SA_KERNEL_MERGE, st);
        hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(n_rows * kLH)), dim3(kLDv / 4), 0, st, vis, sel,
                           split_rows, n_splits, part_o, part_ml, out, lse);
        return hipGetLastError();
    }
    const sa_config_t &c = h.cfg;
    const size_t lds = (size_t)(c.d_qk + c.max_topk) * sizeof(float);
    dim3 grid((unsigned)n_rows, (unsigned)c.n_heads);
    KernelTimer timer(h, SA_KERNEL_ATTENTION, st);
    if (c.dtype == SA_BF16)
        hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(256), lds, st,
                           reinterpret_cast<const uint16_t *>(q), c.n_heads, c.n_kv_heads, c.d_qk, c.d_v,
                           kv, v, vis, sel, scale_log2, out, lse, h.d_err);
    else
        hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(256), lds, st,
                           reinterpret_cast<const float *>(q), c.n_heads, c.n_kv_heads, c.d_qk, c.d_v,
                           kv, v, vis, sel, scale_log2, out, lse, h.d_err);
    return hipGetLastError();
}

}  // namespace sa
