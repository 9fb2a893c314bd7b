// Lightning-indexer scores on gfx950.
//
// I(t,s) = sum_j w(t,j) * ReLU( q(t,j) . k(s) ) over H_I index heads of width d_I with one
// index key per token -- "Sparse Attention and RL Optimization: Three Technical
// Breakthroughs in LLM Post-Training", section 2.2; keys after the query's visible range
// are masked to -inf (section 2.5 pseudocode: only look-back is allowed).
//
// Two kernels:
//  * indexer_mfma_kernel (bf16, H_I = 64, d_I = 128): the contraction over d_I is a dense
//    [64 heads x 128] . [128 x 32 keys] product per query, issued as 16
//    v_mfma_f32_32x32x16_bf16 per 32-key tile with fp32 accumulation.  The ReLU, the
//    weighting by w and the sum over heads run in the epilogue: each lane owns one key
//    column and 16 head rows of each 32-head tile, so 32 of the 64 head terms are summed
//    in registers and one cross-lane add (lane ^ 32) completes the head sum.
//  * indexer_generic_kernel (any shape, fp32 or bf16): one thread per (query, key).
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

// Pointer to token s of the sequence that query row b belongs to.
template <class T>
__device__ __forceinline__ const T *token_row(const RowSource &src, int64_t b, int64_t s, bool &ok)
{
    if (!src.block_table) {
        ok = true;
        return reinterpret_cast<const T *>(src.base) + s * src.row_elems;
    }
    int32_t page = src.block_table[src.seq_of(b) * src.max_blocks + s / src.page_size];
    ok = page >= 0 && page < src.n_pages;
    if (!ok) page = 0;
    return reinterpret_cast<const T *>(src.base) +
           ((int64_t)page * src.page_size + s % src.page_size) * src.row_elems;
}

constexpr int kHeadsI = 64;   // index heads served by the MFMA kernel
constexpr int kDimI = 128;    // index head width served by the MFMA kernel
constexpr int kKeysPerWG = 128;

// One wave per query row, four rows per workgroup, 128 keys per workgroup (4 tiles of 32).
__global__ __launch_bounds__(256) void indexer_mfma_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w, int64_t n_rows,
    RowSource keys, Visibility vis, float *__restrict__ scores, int64_t ld, int64_t n_cols,
    uint32_t *err)
{
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t r = (int64_t)blockIdx.y * 4 + wave;
    if (r >= n_rows) return;
    const int64_t visible = visible_len(vis, r, lane == 0 ? err : nullptr);
    const int64_t s_base = (int64_t)blockIdx.x * kKeysPerWG;
    float *out_row = scores + r * ld;
    const float neg_inf = -__builtin_inff();

    if (s_base >= visible) {
        for (int i = lane; i < kKeysPerWG; i += kWave) {
            int64_t s = s_base + i;
            if (s < n_cols) out_row[s] = neg_inf;
        }
        return;
    }

    // A operand: q(t, head) rows, 8 consecutive bf16 of the d_I axis per lane and k-step.
    // Lane l holds head (32*mt + l%32), dims 16*ks + 8*(l/32) .. +7.
    bf16x8 a[2][kDimI / 16];
    const uint16_t *qr = q_idx + r * kHeadsI * kDimI;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ks = 0; ks < kDimI / 16; ++ks)
            a[mt][ks] = as_bf16x8(load16(qr + (32 * mt + lane % 32) * kDimI + 16 * ks + 8 * (lane / 32)));

    // Head weights in the accumulator layout of v_mfma_f32_32x32x16: register g of lane l
    // holds output row 8*(g/4) + 4*(l/32) + g%4 (a head), column l%32 (a key).
    float wv[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int g = 0; g < 16; ++g)
            wv[mt][g] = w[r * kHeadsI + 32 * mt + 8 * (g / 4) + 4 * (lane / 32) + g % 4];

#pragma unroll 1
    for (int sub = 0; sub < kKeysPerWG / 32; ++sub) {
        const int64_t s0 = s_base + 32 * sub;
        if (s0 >= n_cols) break;
        const int64_t s = s0 + lane % 32;
        if (s0 >= visible) {
            if (lane < 32 && s < n_cols) out_row[s] = neg_inf;
            continue;
        }
        const int64_t s_load = s < visible ? s : visible - 1;
        bool ok;
        const uint16_t *kr = token_row<uint16_t>(keys, r, s_load, ok);
        // B operand: key row s, the same 8 dims per lane as the A operand.
        bf16x8 b[kDimI / 16];
#pragma unroll
        for (int ks = 0; ks < kDimI / 16; ++ks) b[ks] = as_bf16x8(load16(kr + 16 * ks + 8 * (lane / 32)));

        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < kDimI / 16; ++ks) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][ks], b[ks], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][ks], b[ks], acc1, 0, 0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            part = fmaf(wv[0][g], fmaxf(acc0[g], 0.f), part);
            part = fmaf(wv[1][g], fmaxf(acc1[g], 0.f), part);
        }
        part += __shfl_xor(part, 32);
        if (s < visible && !ok && lane < 32) flag_error(err, SA_DEVERR_BLOCK_TABLE);
        if (lane < 32 && s < n_cols) out_row[s] = (s < visible && ok) ? part : neg_inf;
    }
}

// Any H_I, d_I, fp32 or bf16 elements: one thread per (query row, key).
template <class T>
__global__ __launch_bounds__(256) void indexer_generic_kernel(
    const T *__restrict__ q_idx, const float *__restrict__ w, int64_t n_rows, int H_I, int d_I,
    RowSource keys, Visibility vis, float *__restrict__ scores, int64_t ld, int64_t n_cols,
    uint32_t *err)
{
    extern __shared__ float smem[];
    float *qs = smem;                  // [H_I * d_I]
    float *ws = smem + H_I * d_I;      // [H_I]
    const int64_t r = blockIdx.y;
    const int64_t visible = visible_len(vis, r, threadIdx.x == 0 && blockIdx.x == 0 ? err : nullptr);
    for (int i = threadIdx.x; i < H_I * d_I; i += blockDim.x)
        qs[i] = load_elem(q_idx + r * H_I * d_I + i);
    for (int i = threadIdx.x; i < H_I; i += blockDim.x) ws[i] = w[r * H_I + i];
    __syncthreads();
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n_cols) return;
    float score = -__builtin_inff();
    if (s < visible) {
        bool ok;
        const T *kr = token_row<T>(keys, r, s, ok);
        if (ok) {
            score = 0.f;
            for (int j = 0; j < H_I; ++j) {
                float dot = 0.f;
                for (int c = 0; c < d_I; ++c) dot = fmaf(qs[j * d_I + c], load_elem(kr + c), dot);
                score = fmaf(ws[j], fmaxf(dot, 0.f), score);
            }
        } else {
            flag_error(err, SA_DEVERR_BLOCK_TABLE);
        }
    }
    scores[r * ld + s] = score;
}

}  // namespace

hipError_t launch_indexer(sa_handle_s &h, const void *q_idx, const float *w,
                          int64_t n_rows, RowSource keys, Visibility vis, float *scores,
                          int64_t ld, int64_t n_cols, hipStream_t st)
{
    if (n_rows <= 0 || n_cols <= 0) return hipSuccess;
    KernelTimer timer(h, SA_KERNEL_INDEXER, st);
    if (h.fast_indexer) {
        dim3 grid((unsigned)((n_cols + kKeysPerWG - 1) / kKeysPerWG), (unsigned)((n_rows + 3) / 4));
        hipLaunchKernelGGL(indexer_mfma_kernel, grid, dim3(256), 0, st,
                           reinterpret_cast<const uint16_t *>(q_idx), w, n_rows, keys, vis, scores,
                           ld, n_cols, h.d_err);
    } else {
        const int H_I = h.cfg.n_idx_heads, d_I = h.cfg.d_idx;
        size_t lds = (size_t)(H_I * d_I + H_I) * sizeof(float);
        dim3 grid((unsigned)((n_cols + 255) / 256), (unsigned)n_rows);
        if (h.cfg.dtype == SA_BF16)
            hipLaunchKernelGGL(indexer_generic_kernel<uint16_t>, grid, dim3(256), lds, st,
                               reinterpret_cast<const uint16_t *>(q_idx), w, n_rows, H_I, d_I, keys,
                               vis, scores, ld, n_cols, h.d_err);
        else
            hipLaunchKernelGGL(indexer_generic_kernel<float>, grid, dim3(256), lds, st,
                               reinterpret_cast<const float *>(q_idx), w, n_rows, H_I, d_I, keys,
                               vis, scores, ld, n_cols, h.d_err);
    }
    return hipGetLastError();
}

}  // namespace sa
