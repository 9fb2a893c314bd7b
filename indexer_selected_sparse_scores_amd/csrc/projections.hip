// Index-space projections on gfx950: the first two lines of the pseudocode in "Sparse Attention
// and RL Optimization: Three Technical Breakthroughs in LLM Post-Training", section 2.5 -- the
// index query and key are linear maps of the attention query and key (i_q = W_iq(q),
// i_k = W_ik(k)).  The head weights w(t, j) of the score in section 2.2 are taken as one more
// linear map of the query row.
//
//  * q side: q_idx = q W_iq^T (bf16 out) and w = q W_w^T (fp32 out) are plain GEMMs over the
//    H * d_qk query row (9216 wide for the latent shapes): they run on hipBLASLt, bf16 inputs
//    with fp32 accumulation.
//  * k side: k_idx = k W_ik^T over the 576-wide latent row, one v_mfma_f32_32x32x16_bf16 tile
//    of 32 tokens x 32 index dims per wave, written straight to its destination row: the
//    contiguous [L, d_I] array, or the token's slot of the paged index-key cache.
#include <hipblaslt/hipblaslt.h>

#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

namespace {

constexpr int kPD = 128;                 // index dims (d_I) of the key projection kernel
constexpr int kPRows = 32;               // tokens per workgroup
constexpr int kPThreads = 4 * kWave;     // wave w makes index dims 32 w .. 32 w + 31
constexpr int kTileLd = kPD + 8;         // padded LDS row of the output tile (bf16)

// k_idx of tokens r0 .. r0 + 31.  A operand: token r0 + l % 32 (clamped to the last row),
// k-elements 16 s + 8 (l / 32) .. +7; B operand: W_ik row 32 w + l % 32 (index dim), same
// k-elements.  The fp32 tile is rounded to bf16 and staged in LDS, then written as whole
// 256-byte rows: contiguous, or to page block_table[seq, pos / page_size], slot
// pos % page_size, with (seq, pos) = (row_seq[r], row_pos[r]), defaulting to (0, pos0 + r); a row whose
// sequence, position or page entry is out of range is skipped and flagged.
__global__ __launch_bounds__(kPThreads) void project_k_kernel(
    const uint16_t *__restrict__ k, int64_t L, int K, const uint16_t *__restrict__ W, uint16_t *__restrict__ out,
    const int32_t *__restrict__ block_table, int32_t n_seqs, int32_t max_blocks, int32_t page_size, int64_t n_pages,
    const int32_t *__restrict__ row_seq, const int32_t *__restrict__ row_pos, int64_t pos0, uint32_t *err)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[kPRows][kTileLd];
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int64_t r0 = (int64_t)blockIdx.x * kPRows;
    int64_t arow = r0 + lane % 32;
    if (arow >= L) arow = L - 1;
    const uint16_t *ap = k + arow * (int64_t)K + 8 * (lane / 32);
    const uint16_t *bp = W + (int64_t)(32 * wave + lane % 32) * K + 8 * (lane / 32);
    f32x16 acc = {};
#pragma unroll 6
    for (int s = 0; s < K / 16; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(load16(ap + 16 * s)), as_bf16x8(load16(bp + 16 * s)),
                                                      acc, 0, 0, 0);
    // register i of lane l: token 8 (i / 4) + 4 (l / 32) + i % 4, index dim 32 wave + l % 32
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const __bf16 v = (__bf16)acc[i];
        tile[8 * (i / 4) + 4 * (lane / 32) + i % 4][32 * wave + lane % 32] = __builtin_bit_cast(uint16_t, v);
    }
    __syncthreads();
    // thread t writes bytes 32 (t % 8) .. +31 of token row t / 8
    const int row = tid / 8, part = tid % 8;
    const int64_t r = r0 + row;
    if (r >= L) return;
    uint16_t *dst;
    if (!block_table) {
        dst = out + r * kPD;
    } else {
        const int64_t seq = row_seq ? row_seq[r] : 0;
        const int64_t pos = row_pos ? (int64_t)row_pos[r] : pos0 + r;
        const int64_t lp = pos >= 0 ? pos / page_size : -1;
        const int32_t page = lp >= 0 && lp < max_blocks && seq >= 0 && seq < n_seqs ? block_table[seq * max_blocks + lp] : -1;
        if (page < 0 || page >= n_pages) {
            if (part == 0) flag_error(err, SA_DEVERR_BLOCK_TABLE);
            return;
        }
        dst = out + ((int64_t)page * page_size + pos % page_size) * kPD;
    }
    const uint4 *src = reinterpret_cast<const uint4 *>(&tile[row][16 * part]);
    uint4 *d = reinterpret_cast<uint4 *>(dst + 16 * part);
    d[0] = src[0];
    d[1] = src[1];
}

struct BltState {
    hipblasLtHandle_t lt = nullptr;
};

const char *blt_name(hipblasStatus_t s)
{
    switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialised";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    default: return "error";
    }
}

// Y [L, N] = X [L, K] W [N, K]^T, row-major, bf16 inputs, fp32 accumulation, output bf16 or
// fp32.  In hipBLASLt's column-major terms: D (N x L, ld N) = A^T B with A = W (K x N, ld K)
// and B = X (K x L, ld K).
sa_status_t gemm_tn(sa_handle_s &h, hipblasLtHandle_t lt, const void *X, const void *W, void *Y, int64_t L,
                    int64_t K, int64_t N, bool out_bf16, void *ws, size_t ws_bytes, hipStream_t st)
{
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    hipblasStatus_t s = hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    const uint64_t wsb = ws_bytes;
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, K, N, K);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, K, L, K);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&ld, out_bf16 ? HIP_R_16BF : HIP_R_32F, N, L, N);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulPreferenceCreate(&pref);
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));
    hipblasLtMatmulHeuristicResult_t res{};
    int count = 0;
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulAlgoGetHeuristic(lt, desc, la, lb, ld, ld, pref, 1, &res, &count);
    if (s == HIPBLAS_STATUS_SUCCESS && count < 1) s = HIPBLAS_STATUS_NOT_SUPPORTED;
    const float alpha = 1.f, beta = 0.f;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmul(lt, desc, &alpha, W, la, X, lb, &beta, Y, ld, Y, ld, &res.algo, ws, ws_bytes, st);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (ld) hipblasLtMatrixLayoutDestroy(ld);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (desc) hipblasLtMatmulDescDestroy(desc);
    if (s != HIPBLAS_STATUS_SUCCESS) {
        h.last_error = std::string("hipBLASLt GEMM (") + std::to_string(L) + " x " + std::to_string(N) + " x " +
                       std::to_string(K) + "): " + blt_name(s);
        return SA_ERR_HIP;
    }
    return SA_OK;
}

}  // namespace

size_t projection_workspace() { return size_t(32) << 20; }

sa_status_t launch_project_q(sa_handle_s &h, const void *q, int64_t L, const void *W_iq, const void *W_w,
                             void *q_idx, float *w, void *ws, size_t ws_bytes, hipStream_t st)
{
    BltState *b = static_cast<BltState *>(h.blt);
    if (!b) {
        b = new BltState;
        const hipblasStatus_t s = hipblasLtCreate(&b->lt);
        if (s != HIPBLAS_STATUS_SUCCESS) {
            delete b;
            h.last_error = std::string("hipblasLtCreate: ") + blt_name(s);
            return SA_ERR_HIP;
        }
        h.blt = b;
    }
    const int64_t K = (int64_t)h.cfg.n_heads * h.cfg.d_qk;
    sa_status_t s = SA_OK;
    if (W_iq) {
        KernelTimer timer(h, SA_KERNEL_PROJECT, st);
        s = gemm_tn(h, b->lt, q, W_iq, q_idx, L, K, (int64_t)h.cfg.n_idx_heads * h.cfg.d_idx, true, ws, ws_bytes, st);
    }
    if (s == SA_OK && W_w) {
        KernelTimer timer(h, SA_KERNEL_PROJECT, st);
        s = gemm_tn(h, b->lt, q, W_w, w, L, K, h.cfg.n_idx_heads, false, ws, ws_bytes, st);
    }
    return s;
}

hipError_t launch_project_k(sa_handle_s &h, const void *k, int64_t L, const void *W_ik, void *k_idx,
                            const int32_t *block_table, int32_t n_seqs, int32_t max_blocks, int64_t n_pages,
                            const int32_t *row_seq, const int32_t *row_pos, int64_t pos0, hipStream_t st)
{
    const int K = h.cfg.n_kv_heads * h.cfg.d_qk;
    KernelTimer timer(h, SA_KERNEL_PROJECT, st);
    hipLaunchKernelGGL(project_k_kernel, dim3((unsigned)((L + kPRows - 1) / kPRows)), dim3(kPThreads), 0, st,
                       reinterpret_cast<const uint16_t *>(k), L, K, reinterpret_cast<const uint16_t *>(W_ik),
                       reinterpret_cast<uint16_t *>(k_idx), block_table, n_seqs, max_blocks, h.cfg.page_size, n_pages,
                       row_seq, row_pos, pos0, h.d_err);
    return hipGetLastError();
}

void destroy_projection_state(sa_handle_s &h)
{
    BltState *b = static_cast<BltState *>(h.blt);
    if (!b) return;
    if (b->lt) hipblasLtDestroy(b->lt);
    delete b;
    h.blt = nullptr;
}

}  // namespace sa
