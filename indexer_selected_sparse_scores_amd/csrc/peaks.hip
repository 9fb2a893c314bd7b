// Peaks measured on the device, the denominators beside the published ones in the rooflines: a bf16
// MFMA loop on random operands (with the shader clock it ran at) and streaming read / copy kernels.
// Measurement aids only: nothing of the method runs here.
//
// peak_mfma_kernel runs the instruction and the occupancy of the fused prefill indexer -- eight waves
// per compute unit (two per SIMD), v_mfma_f32_32x32x16_bf16 with fp32 accumulation -- with operands that
// change at every MFMA (eight different random A / B fragment pairs per wave, cycled), since the
// multipliers' switching, and so the power-limited clock, depends on the data.  Thread 0 of each
// workgroup reads the shader-clock counter (s_memtime) and the 100 MHz reference counter
// (s_memrealtime) around the loop, so the host can tell the clock the loop ran at.
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

namespace {

constexpr int kPeakThreads = 512;  // eight waves: two per SIMD
constexpr int kPeakSets = 8;       // operand pairs per wave, one per MFMA of an iteration
constexpr int kPeakChains = 4;     // independent accumulators
constexpr int kPeakOperandWaves = 64;  // distinct operand blocks in the caller's buffer (waves share them cyclically)
constexpr int kPeakClockBlocks = 64;   // workgroups whose clock counters are kept
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;      // 16-byte loads in flight per thread
constexpr int kPeakStreamBlocksPerCu = 8;

__global__ __launch_bounds__(kPeakThreads, 1) void peak_mfma_kernel(const uint4 *__restrict__ operands, int iters,
                                                                      unsigned long long *__restrict__ clocks,
                                                                      float *__restrict__ sink)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const uint4 *src = operands + (size_t)((blockIdx.x * (kPeakThreads / kWave) + wave) % kPeakOperandWaves) *
                                      (2 * kPeakSets * kWave);
    bf16x8 a[kPeakSets], b[kPeakSets];
#pragma unroll
    for (int i = 0; i < kPeakSets; ++i) {
        a[i] = as_bf16x8(src[(2 * i) * kWave + lane]);
        b[i] = as_bf16x8(src[(2 * i + 1) * kWave + lane]);
    }
    f32x16 acc[kPeakChains];
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) acc[c] = f32x16{};
    __syncthreads();
    unsigned long long t0 = 0, r0 = 0;
    if (tid == 0) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kPeakSets; ++i)
            acc[i % kPeakChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], acc[i % kPeakChains], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[c][j];
    if (s == 1234.5f) sink[0] = s;  // keeps the loop's results live
    __syncthreads();
    if (tid == 0 && blockIdx.x < kPeakClockBlocks) {
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        clocks[4 * blockIdx.x + 0] = t0;
        clocks[4 * blockIdx.x + 1] = t1;
        clocks[4 * blockIdx.x + 2] = r0;
        clocks[4 * blockIdx.x + 3] = r1;
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming read (dst == nullptr: every 16 bytes of src is loaded once and folded into one value per
// thread) or copy (dst != nullptr) of n4 16-byte words, grid-stride, kStreamUnroll loads in flight.
__global__ __launch_bounds__(kStreamThreads) void peak_stream_kernel(const u32x4 *__restrict__ src,
                                                                     u32x4 *__restrict__ dst, int64_t n4,
                                                                     float *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    uint32_t fold = 0;
    int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    for (; i + (kStreamUnroll - 1) * stride < n4; i += kStreamUnroll * stride) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            if (dst)
                __builtin_nontemporal_store(v[u], dst + i + u * stride);
            else
                fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    for (; i < n4; i += stride) {
        const u32x4 v = src[i];
        if (dst)
            dst[i] = v;
        else
            fold ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (!dst && fold == 0x9E3779B9u) sink[0] = __uint_as_float(fold);  // keeps the loads live
}

}  // namespace

}  // namespace sa

namespace {

sa_status_t peak_fail(sa_handle_t h, sa_status_t st, const char *msg)
{
    if (h) h->last_error = msg;
    return st;
}

}  // namespace

extern "C" {

sa_status_t sparse_attn_peak_mfma(sa_handle_t h, const void *operands, int32_t iters, uint64_t *clocks, float *sink,
                                  void *stream)
{
    if (!h) return SA_ERR_INVALID_ARG;
    h->last_error.clear();
    if (!operands || !clocks || !sink) return peak_fail(h, SA_ERR_INVALID_ARG, "NULL pointer");
    if (iters < 1) return peak_fail(h, SA_ERR_INVALID_ARG, "iters must be >= 1");
    if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0)
        return peak_fail(h, SA_ERR_INVALID_ARG, "operands must be 16-byte aligned");
    if (h->device < 0) return peak_fail(h, SA_ERR_UNSUPPORTED, "a host-only handle launches nothing");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
        return peak_fail(h, SA_ERR_INVALID_ARG, "the current device is not the handle's device");
    hipLaunchKernelGGL(sa::peak_mfma_kernel, dim3((unsigned)h->n_cu), dim3(sa::kPeakThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4 *>(operands), (int)iters,
                       reinterpret_cast<unsigned long long *>(clocks), sink);
    return hipGetLastError() == hipSuccess ? SA_OK : peak_fail(h, SA_ERR_HIP, "peak MFMA launch failed");
}

sa_status_t sparse_attn_peak_stream(sa_handle_t h, const void *src, void *dst, int64_t bytes, float *sink,
                                    void *stream)
{
    if (!h) return SA_ERR_INVALID_ARG;
    h->last_error.clear();
    if (!src || (!dst && !sink)) return peak_fail(h, SA_ERR_INVALID_ARG, "NULL pointer");
    if (bytes < 16 || (bytes & 15) != 0) return peak_fail(h, SA_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15u) != 0)
        return peak_fail(h, SA_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    if (h->device < 0) return peak_fail(h, SA_ERR_UNSUPPORTED, "a host-only handle launches nothing");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
        return peak_fail(h, SA_ERR_INVALID_ARG, "the current device is not the handle's device");
    hipLaunchKernelGGL(sa::peak_stream_kernel, dim3((unsigned)(h->n_cu * sa::kPeakStreamBlocksPerCu)),
                       dim3(sa::kStreamThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const sa::u32x4 *>(src), reinterpret_cast<sa::u32x4 *>(dst), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? SA_OK : peak_fail(h, SA_ERR_HIP, "peak stream launch failed");
}

}  // extern "C"
