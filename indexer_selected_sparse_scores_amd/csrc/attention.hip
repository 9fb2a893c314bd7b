// Softmax attention over the indexer-selected rows on gfx950.
//
// For query row r and head h: O = sum_{s in sel(r)} softmax_s(scale q_h . K_s) V_s -- the
// "execute main attention only on selected tokens" step of "Sparse Attention and RL
// Optimization: Three Technical Breakthroughs in LLM Post-Training", section 2.5, and of
// "Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and
// Verifiable Synthetic Data", section 2.4.  In decode only the selected rows of the paged
// cache are read (that page, section 2.3).
//
// attn_latent_mfma_kernel serves the latent layout (bf16, 16 heads sharing one 576-wide
// row per token whose first 512 columns are the value).  A 256-thread workgroup gathers 64
// selected rows at a time into LDS with 16-byte loads (1152 bytes per row, read once for
// all 16 heads), computes the 16 x 64 logits with v_mfma_f32_16x16x32_bf16 (each wave
// takes 16 rows), keeps an online softmax (running max / sum per head, exp2 with the log2(e)
// factor folded into the scale), and accumulates P.V with the same MFMA, each wave owning
// 128 of the 512 value columns.  P enters the MFMA as a bf16 hi part plus a bf16 residual,
// so the weights keep ~16 mantissa bits.  In decode the selected rows of one sequence are
// split across workgroups and a second kernel merges the partial (max, sum, accumulator)
// states.
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

// Element offset of token s of the sequence of query row b, or -1 if its page is invalid.
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
constexpr int kChunk = 64;      // selected rows per LDS chunk
constexpr int kRowBytes = kLDqk * 2;
constexpr int kLdsRow = kRowBytes + 16;   // padded LDS row stride (bytes)
constexpr int kPieces = kRowBytes / 16;   // 16-byte pieces per row
constexpr int kLoadIters = kChunk * kPieces / 256;
static_assert(kChunk * kPieces % 256 == 0, "chunk load must tile the workgroup");

template <bool kSplit>
__global__ __launch_bounds__(256, 2) void attn_latent_mfma_kernel(
    const uint16_t *__restrict__ q, int64_t n_rows, RowSource kv, Visibility vis, Selection sel,
    float scale_log2, float *__restrict__ out, float *__restrict__ lse, int split_rows, int n_splits,
    float *__restrict__ part_o, float *__restrict__ part_ml, uint32_t *err)
{
    __shared__ __attribute__((aligned(16))) unsigned char rows_lds[kChunk * kLdsRow];
    __shared__ float s_lds[kLH * kChunk];
    __shared__ int64_t row_off[kChunk];

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int hh = lane % 16, grp = lane / 16;
    const int64_t r = blockIdx.x;
    const int split = kSplit ? (int)blockIdx.y : 0;
    uint32_t *err0 = (tid == 0 && split == 0) ? err : nullptr;
    const int64_t visible = visible_len(vis, r, err0);
    const int64_t kr = budget(sel, r, err0);
    const int64_t m = kr < visible ? kr : visible;
    const int64_t j_begin = kSplit ? (int64_t)split * split_rows : 0;
    const int64_t j_end = kSplit ? (j_begin + split_rows < m ? j_begin + split_rows : m) : m;
    if (kSplit && j_begin >= m) return;  // the merge kernel ignores unused splits
    const int32_t *idx_row = sel.idx + r * sel.idx_ld;
    const uint16_t *kv_base = reinterpret_cast<const uint16_t *>(kv.base);

    // A operand of Q.K^T: head hh, dims 32*ks + 8*grp .. +7
    bf16x8 qa[kLDqk / 32];
    const uint16_t *qr = q + (r * kLH + hh) * kLDqk;
#pragma unroll
    for (int ks = 0; ks < kLDqk / 32; ++ks) qa[ks] = as_bf16x8(load16(qr + 32 * ks + 8 * grp));

    const float neg_inf = -__builtin_inff();
    float m_run = neg_inf, l_run = 0.f;   // softmax state of head hh (log2 domain)
    f32x4 acc[8];                         // O[4*grp + i][128*wave + 16*nt + hh]
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
    for (int64_t c = j_begin; c < j_end; c += kChunk) {
        if (tid < kChunk) {
            int64_t j = c + tid, off = -1;
            if (j < j_end) {
                int64_t s = idx_row[j];
                if (s >= visible) flag_error(err, SA_DEVERR_INDEX_RANGE);
                if (s >= 0 && s < visible) {
                    off = token_offset(kv, r, s);
                    if (off < 0) flag_error(err, SA_DEVERR_BLOCK_TABLE);
                }
            }
            row_off[tid] = off;
        }
        __syncthreads();
        // gather the chunk: 64 rows x 72 pieces of 16 bytes, zero rows for unused slots
#pragma unroll
        for (int it = 0; it < kLoadIters; ++it) {
            const int p = tid + 256 * it;
            const int row = p / kPieces, piece = p % kPieces;
            const int64_t off = row_off[row];
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (off >= 0) v = load16(kv_base + off + piece * 8);
            *reinterpret_cast<uint4 *>(rows_lds + row * kLdsRow + piece * 16) = v;
        }
        __syncthreads();

        // logits of rows 16*wave .. +15 for all 16 heads
        {
            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
            const unsigned char *kb = rows_lds + (16 * wave + hh) * kLdsRow + 16 * grp;
#pragma unroll
            for (int ks = 0; ks < kLDqk / 32; ++ks) {
                bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4 *>(kb + 64 * ks));
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], b, sacc, 0, 0, 0);
            }
            const int row = 16 * wave + hh;
            const bool valid = row_off[row] >= 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_lds[(4 * grp + i) * kChunk + row] = valid ? sacc[i] * scale_log2 : neg_inf;
        }
        __syncthreads();

        // online softmax update for head hh over the 64 rows (identical in every wave)
        float p[16];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) p[8 * ks + i] = s_lds[hh * kChunk + 32 * ks + 8 * grp + i];
        float cmax = p[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) cmax = fmaxf(cmax, p[i]);
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        const float m_new = fmaxf(m_run, cmax);
        const bool any = m_new != neg_inf;
        const float alpha = any ? exp2f(m_run - m_new) : 1.f;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = any ? exp2f(p[i] - m_new) : 0.f;
            psum += p[i];
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;

        bf16x8 pa_hi[2], pa_lo[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint16_t hi[8], lo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                hi[i] = f32_to_bf16_bits(p[8 * ks + i]);
                lo[i] = f32_to_bf16_bits(p[8 * ks + i] - bf16_bits_to_f32(hi[i]));
            }
            uint4 vh = make_uint4(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16),
                                  hi[4] | ((uint32_t)hi[5] << 16), hi[6] | ((uint32_t)hi[7] << 16));
            uint4 vl = make_uint4(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16),
                                  lo[4] | ((uint32_t)lo[5] << 16), lo[6] | ((uint32_t)lo[7] << 16));
            pa_hi[ks] = as_bf16x8(vh);
            pa_lo[ks] = as_bf16x8(vl);
        }
        // rescale the accumulator rows (heads 4*grp + i) by their alpha
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = __shfl(alpha, 4 * grp + i);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[nt][i] *= a;
        }
        // P.V over the 64 rows; V[row][col] is column col of the gathered latent row
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int col = 128 * wave + 16 * nt + hh;
                const unsigned char *vb = rows_lds + (32 * ks + 8 * grp) * kLdsRow + 2 * col;
                uint16_t e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = *reinterpret_cast<const uint16_t *>(vb + i * kLdsRow);
                uint4 vv = make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                                      e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16));
                const bf16x8 b = as_bf16x8(vv);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi[ks], b, acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo[ks], b, acc[nt], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    if (!kSplit) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float iv = __shfl(inv, 4 * grp + i);
            float *orow = out + (r * kLH + 4 * grp + i) * kLDv + 128 * wave + hh;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) orow[16 * nt] = acc[nt][i] * iv;
        }
        if (lse && wave == 0 && lane < kLH)
            lse[r * kLH + lane] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : neg_inf;
    } else {
        const int64_t slot = r * n_splits + split;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *prow = part_o + (slot * kLH + 4 * grp + i) * kLDv + 128 * wave + hh;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) prow[16 * nt] = acc[nt][i];
        }
        if (wave == 0 && lane < kLH) {
            part_ml[(slot * kLH + lane) * 2 + 0] = m_run;
            part_ml[(slot * kLH + lane) * 2 + 1] = l_run;
        }
    }
}

// Merge the per-split softmax states of each decode row: O = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s with M = max_s m_s.
__global__ __launch_bounds__(256) void attn_merge_kernel(
    Visibility vis, Selection sel, int split_rows, int n_splits, int H, int d_v,
    const float *__restrict__ part_o, const float *__restrict__ part_ml, float *__restrict__ out,
    float *__restrict__ lse)
{
    const int64_t r = blockIdx.x;
    int64_t visible = vis.ctx_len ? (int64_t)vis.ctx_len[r] : vis.causal_row0 + r + 1;
    if (vis.ctx_len && (visible < 1 || visible > vis.max_ctx)) visible = 0;
    int64_t k = sel.k_per_row ? (int64_t)sel.k_per_row[r] : (int64_t)sel.k;
    if (k < 1 || k > sel.k) k = 0;
    const int64_t m = k < visible ? k : visible;
    const int used = (int)((m + split_rows - 1) / split_rows);
    const float neg_inf = -__builtin_inff();
    for (int e = threadIdx.x; e < H * d_v; e += blockDim.x) {
        const int h = e / d_v, d = e % d_v;
        float M = neg_inf;
        for (int s = 0; s < used; ++s) M = fmaxf(M, part_ml[((r * n_splits + s) * H + h) * 2]);
        float num = 0.f, den = 0.f;
        if (M != neg_inf) {
            for (int s = 0; s < used; ++s) {
                const int64_t slot = (r * n_splits + s) * H + h;
                const float ms = part_ml[slot * 2];
                if (ms == neg_inf) continue;
                const float f = exp2f(ms - M);
                den = fmaf(part_ml[slot * 2 + 1], f, den);
                num = fmaf(part_o[slot * d_v + d], f, num);
            }
        }
        out[(r * H + h) * (int64_t)d_v + d] = den > 0.f ? num / den : 0.f;
        if (lse && d == 0) lse[r * H + h] = den > 0.f ? (M + __log2f(den)) * kLn2 : neg_inf;
    }
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
    for (int c = threadIdx.x; c < d_qk; c += blockDim.x) qh[c] = load_elem(q + (r * H + h) * (int64_t)d_qk + c);
    __syncthreads();

    const float neg_inf = -__builtin_inff();
    float mx = neg_inf;
    for (int64_t j = threadIdx.x; j < m; j += blockDim.x) {
        const int64_t s = idx_row[j];
        float l = neg_inf;
        if (s >= visible && h == 0) flag_error(err, SA_DEVERR_INDEX_RANGE);
        if (s >= 0 && s < visible) {
            const int64_t off = token_offset(kv, r, s);
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
            const int64_t off = token_offset(vbase ? vsrc : kv, r, s);
            const T *vr = vbase ? vbase + off + (int64_t)g * d_v : kbase + off + (int64_t)g * d_qk;
            a = fmaf(p, load_elem(vr + d), a);
        }
        out[(r * H + h) * (int64_t)d_v + d] = sum > 0.f ? a / sum : 0.f;
    }
    if (lse && threadIdx.x == 0) lse[r * H + h] = sum > 0.f ? (mx + __log2f(sum)) * kLn2 : neg_inf;
}

constexpr int kSplitRows = 256;

}  // namespace

size_t attention_workspace(const sa_handle_s &h, int64_t n_rows, bool decode)
{
    if (!decode || !h.fast_attn) return 0;
    const int64_t n_splits = (h.cfg.max_topk + kSplitRows - 1) / kSplitRows;
    return (size_t)n_rows * n_splits * kLH * (kLDv + 2) * sizeof(float);
}

hipError_t launch_attention(sa_handle_s &h, const void *q, int64_t n_rows, RowSource kv,
                            RowSource v, Visibility vis, Selection sel, float *out, float *lse,
                            void *ws, hipStream_t st)
{
    if (n_rows <= 0) return hipSuccess;
    const float scale_log2 = h.scale * kLog2e;
    const bool decode = vis.ctx_len != nullptr;
    if (h.fast_attn) {
        const uint16_t *qq = reinterpret_cast<const uint16_t *>(q);
        if (!decode) {
            KernelTimer timer(h, SA_KERNEL_ATTENTION, st);
            hipLaunchKernelGGL(attn_latent_mfma_kernel<false>, dim3((unsigned)n_rows), dim3(256), 0, st,
                               qq, n_rows, kv, vis, sel, scale_log2, out, lse, 0, 1, nullptr, nullptr,
                               h.d_err);
            return hipGetLastError();
        }
        const int n_splits = (h.cfg.max_topk + kSplitRows - 1) / kSplitRows;
        float *part_o = reinterpret_cast<float *>(ws);
        float *part_ml = part_o + (size_t)n_rows * n_splits * kLH * kLDv;
        {
            KernelTimer timer(h, SA_KERNEL_ATTENTION, st);
            hipLaunchKernelGGL(attn_latent_mfma_kernel<true>, dim3((unsigned)n_rows, (unsigned)n_splits),
                               dim3(256), 0, st, qq, n_rows, kv, vis, sel, scale_log2, out, lse,
                               kSplitRows, n_splits, part_o, part_ml, h.d_err);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        KernelTimer timer(h, SA_KERNEL_MERGE, st);
        hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)n_rows), dim3(256), 0, st, vis, sel,
                           kSplitRows, n_splits, kLH, kLDv, part_o, part_ml, out, lse);
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
