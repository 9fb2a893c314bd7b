// Index-space projections on gfx950: the first two lines of the pseudocode in "Sparse Attention
// and RL Optimization: Three Technical Breakthroughs in LLM Post-Training", section 2.5 -- the
// index query and key are linear maps of the attention query and key (i_q = W_iq(q),
// i_k = W_ik(k)).  The head weights w(t, j) of the score in section 2.2 are taken as one more
// linear map of the query row.
//
//  * q side: q_idx = q W_iq^T (bf16 out) and w = q W_w^T (fp32 out) are plain GEMMs over the
//    H * d_qk query row (9216 wide for the latent shapes): they run on hipBLASLt, bf16 inputs
//    with fp32 accumulation.
//  * k side: k_idx = k W_ik^T over the 576-wide latent row on v_mfma_f32_32x32x16_bf16, W_ik
//    held in LDS by persistent workgroups, each projected row written straight to where it
//    belongs: the contiguous [L, d_I] array, or the token's slot of the paged index-key cache.
#include <hipblaslt/hipblaslt.h>

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

void destroy_projection_state(sa_handle_s &h)
{
    BltState *b = static_cast<BltState *>(h.blt);
    if (!b) return;
    if (b->lt) hipblasLtDestroy(b->lt);
    delete b;
    h.blt = nullptr;
}

}  // namespace sa
