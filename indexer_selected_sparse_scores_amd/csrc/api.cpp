// C ABI of libsparse_attn: host-side validation, workspace carving and kernel launches.
// Every entry point validates its arguments before launching anything, never allocates
// device memory (except the error word in sparse_attn_create) and never synchronises
// (except sparse_attn_check and sparse_attn_destroy).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>

#include "sa_internal.hpp"

// Device memory of sparse_attn_decode_noalloc, the decode step for callers that cannot allocate: one
// array per device, used in place of a caller workspace.  Host code never passes the array's name (on
// the host it is only a stand-in): it uses the address hipGetSymbolAddress returns on each device, looked
// up once per device when the first handle is created there and kept in g_scratch.  The array sits at
// file scope, outside any unnamed namespace: there its device symbol would be local to the code object,
// and the runtime could not find it by the name the host side registers.
static __device__ __align__(256) unsigned char scratch[size_t(64) << 20];

namespace {

thread_local std::string g_create_error;

constexpr size_t kNoAllocBytes = sizeof(scratch);
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

constexpr int64_t kMaxIndexerScoresL = 16384;
constexpr int32_t kMaxTopk = 8192;
constexpr size_t kAlign = 256;
// Prefill scores are produced and consumed per block of query rows; a block's scores
// take at most this many bytes of workspace.
constexpr size_t kPrefillChunkBytes = size_t(1) << 29;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

sa_status_t fail(sa_handle_t h, sa_status_t st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    if (h) h->last_error = buf;
    else g_create_error = buf;
    return st;
}

sa_status_t hip_status(sa_handle_t h, hipError_t e, const char *what)
{
    if (e == hipSuccess) return SA_OK;
    return fail(h, SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(const sa_handle_s &h) { return h.cfg.dtype == SA_BF16 ? 2 : 4; }

sa_status_t check_device(sa_handle_t h)
{
    if (h->device < 0)
        return fail(h, SA_ERR_UNSUPPORTED,
                    "a host-only handle (sparse_attn_create_host) validates and sizes calls but launches nothing");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(h, SA_ERR_HIP, "hipGetDevice failed");
    if (dev != h->device)
        return fail(h, SA_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev,
                    h->device);
    return SA_OK;
}

// Rows of queries whose scores are materialised at once in the prefill workspace.
int64_t prefill_chunk_rows(int64_t L)
{
    int64_t rows = (int64_t)(kPrefillChunkBytes / (sizeof(float) * (size_t)L));
    rows = rows / 4 * 4;
    if (rows < 4) rows = 4;
    if (rows > L) rows = L;
    return rows;
}

struct PrefillLayout {
    size_t scores, idx, total;
};

// Fast path (bf16, 64 x 128 indexer): [idx | fused indexer/top-k workspace].
// Generic path, and every two-tier selection: [scores of one block of query rows | idx].
PrefillLayout prefill_layout(const sa_handle_s &h, int64_t L, bool chunked = false)
{
    PrefillLayout p;
    if (h.fast_indexer && !chunked) {
        p.idx = 0;
        p.scores = align_up((size_t)L * (size_t)h.cfg.max_topk * sizeof(int32_t));
        p.total = p.scores + align_up(sa::prefill_topk_workspace(h, L));
        return p;
    }
    p.scores = 0;
    p.idx = align_up((size_t)prefill_chunk_rows(L) * (size_t)L * sizeof(float));
    p.total = p.idx + align_up((size_t)L * (size_t)h.cfg.max_topk * sizeof(int32_t));
    return p;
}

// Two-tier prefill on the fused kernels: [idx | tile counter | block keys [L, ceil(L / 64)] uint32].
struct BlocksFusedLayout {
    size_t idx, counter, keys, total;
};

BlocksFusedLayout blocks_fused_layout(const sa_handle_s &h, int64_t L)
{
    BlocksFusedLayout b;
    b.idx = 0;
    b.counter = align_up((size_t)L * (size_t)h.cfg.max_topk * sizeof(int32_t));
    b.keys = b.counter + kAlign;
    b.total = b.keys + align_up((size_t)L * sa::prefill_block_keys_ld(L, 0) * sizeof(uint32_t));
    return b;
}

bool blocks_fused(const sa_handle_s &h, int32_t block_size) { return h.fast_indexer && block_size >= 64; }

struct DecodeLayout {
    size_t scores, idx, attn, total;
};

// Fast path: [decode top-k workspace (scores, histograms, candidates) | idx | attention
// partials].  Generic path: [scores [B, max_ctx] | idx | attention partials].
DecodeLayout decode_layout(const sa_handle_s &h, int64_t B, int64_t max_ctx)
{
    DecodeLayout d;
    d.scores = 0;
    d.idx = h.fast_decode ? align_up(sa::decode_topk_layout(B, max_ctx).total)
                          : align_up((size_t)B * (size_t)max_ctx * sizeof(float));
    d.attn = d.idx + align_up((size_t)B * (size_t)h.cfg.max_topk * sizeof(int32_t));
    d.total = d.attn + align_up(sa::attention_workspace(h, B, true));
    return d;
}

// Query rows against paged caches: [row_seq copy | ctx | budget | scores (and histograms) of one
// block of rows | idx | split-attention partials (few rows only)].
struct PagedLayout {
    size_t seq, ctx, budget, scores, idx, attn, total;
    int64_t chunk;   // query rows scored at once (per-row path)
    bool split;      // attention splits each row's selection over workgroups
    bool fused;      // the rows run as fused prefill row tiles (sorted by sequence and position on the device)
};

PagedLayout paged_layout(const sa_handle_s &h, int64_t T, int64_t max_ctx)
{
    PagedLayout p;
    p.fused = sa::prefill_rows_fused(h, T, (int32_t)max_ctx);
    const int64_t ld = h.fast_decode ? (max_ctx + 63) / 64 * 64 : max_ctx;
    int64_t chunk = (int64_t)(kPrefillChunkBytes / (sizeof(float) * (size_t)ld));
    if (chunk < 1) chunk = 1;
    if (chunk > 65535) chunk = 65535;  // grid y of the indexer kernels
    if (chunk > T) chunk = T;
    p.chunk = chunk;
    p.split = h.fast_attn && T < h.n_cu;
    size_t at = 0;
    p.seq = at;
    at += align_up((size_t)T * sizeof(int32_t));
    p.ctx = at;
    at += align_up((size_t)T * sizeof(int32_t));
    p.budget = at;
    at += align_up((size_t)T * sizeof(int32_t));
    p.scores = at;
    if (p.fused)  // the fused row tiles' workspace (candidate lists, row table)
        at += align_up(sa::prefill_rows_workspace(h, T, (int32_t)max_ctx));
    else
        at += align_up(h.fast_decode ? sa::decode_topk_layout(chunk, max_ctx).total
                                     : (size_t)chunk * (size_t)max_ctx * sizeof(float));
    p.idx = at;
    at += align_up((size_t)T * (size_t)h.cfg.max_topk * sizeof(int32_t));
    p.attn = at;
    at += align_up(p.split ? sa::attention_workspace(h, T, true) : 0);
    p.total = at;
    return p;
}

// Chunked prefill of one sequence (C rows at positions pos0 ..): fused path [idx | fused indexer/top-k
// workspace]; generic path [scores of one block of rows | idx].
bool chunk_fused(const sa_handle_s &h, int64_t pos0, int64_t C)
{
    return h.fast_decode && (pos0 + C + 63) / 64 <= sa::kPrefillMaxPages;
}

PrefillLayout chunk_layout(const sa_handle_s &h, int64_t pos0, int64_t C)
{
    PrefillLayout p;
    const size_t idx_bytes = align_up((size_t)C * (size_t)h.cfg.max_topk * sizeof(int32_t));
    if (chunk_fused(h, pos0, C)) {
        p.idx = 0;
        p.scores = idx_bytes;
        p.total = p.scores + align_up(sa::prefill_topk_workspace(h, C, pos0));
        return p;
    }
    const int64_t n = pos0 + C;
    int64_t rows = (int64_t)(kPrefillChunkBytes / (sizeof(float) * (size_t)n));
    rows = rows < 1 ? 1 : (rows > C ? C : rows);
    p.scores = 0;
    p.idx = align_up((size_t)rows * (size_t)n * sizeof(float));
    p.total = p.idx + idx_bytes;
    return p;
}

// Two-tier (block -> token) selection parameters; nullptr selects plain per-query top-k.
struct BlockSelect {
    int32_t block_size, n_blocks;
};

sa_status_t check_block_select(sa_handle_t h, const BlockSelect &b, int64_t cols)
{
    const int32_t bs = b.block_size;
    if (bs < 1 || bs > 1024 || (bs & (bs - 1)) != 0)
        return fail(h, SA_ERR_INVALID_ARG, "block_size (%d) must be a power of two in [1, 1024]", bs);
    if (b.n_blocks < 1 || b.n_blocks > sa::kBlockSelectMaxKept)
        return fail(h, SA_ERR_INVALID_ARG, "n_blocks (%d) must be in [1, %d]", b.n_blocks, sa::kBlockSelectMaxKept);
    if ((int64_t)b.n_blocks * bs > sa::kBlockSelectMaxItems)
        return fail(h, SA_ERR_UNSUPPORTED, "n_blocks * block_size (%lld) exceeds %d candidate tokens",
                    (long long)b.n_blocks * bs, sa::kBlockSelectMaxItems);
    if ((cols + bs - 1) / bs > sa::kBlockSelectMaxItems)
        return fail(h, SA_ERR_UNSUPPORTED, "%lld tokens make more than %d blocks of %d", (long long)cols,
                    sa::kBlockSelectMaxItems, bs);
    return SA_OK;
}

sa_status_t prefill_impl(sa_handle_t h, const void *q, const void *k, const void *v, const void *q_idx,
                         const float *w, const void *k_idx, int64_t L, int32_t topk, const BlockSelect *blocks,
                         float *out, float *lse, int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

sa_status_t decode_impl(sa_handle_t h, const void *q, const void *q_idx, const float *w, const void *kv_pages,
                        const void *v_pages, const void *kidx_pages, int64_t n_pages, const int32_t *block_table,
                        int32_t max_blocks, const int32_t *ctx_len, const int32_t *topk, int32_t B, int32_t max_ctx,
                        const BlockSelect *blocks, float *out, float *lse, int32_t *idx_out, void *ws,
                        size_t ws_bytes, void *stream);

// A batch of sequences with their new rows contiguous: the fused row tiles need the fast kernels and at
// most kPrefillMaxPages pages per sequence; otherwise the rows run as sparse_attn_prefill_paged's rows.
bool varlen_fused(const sa_handle_s &h, int64_t max_ctx)
{
    return h.fast_decode && (max_ctx + 63) / 64 <= sa::kPrefillMaxPages;
}

// Fused: [row_seq | row_pos | seq | ctx | budget | idx | split-attention partials (few rows) | fused
// indexer/top-k workspace].  Otherwise: [row_seq | row_pos | sparse_attn_prefill_paged's workspace].
struct VarlenApiLayout {
    size_t row_seq, row_pos, seq, ctx, budget, idx, attn, rest, total;
    bool split;
};

VarlenApiLayout varlen_api_layout(const sa_handle_s &h, int64_t T, int64_t max_ctx)
{
    VarlenApiLayout v{};
    const size_t rows = align_up((size_t)T * sizeof(int32_t));
    v.row_seq = 0;
    v.row_pos = rows;
    if (!varlen_fused(h, max_ctx)) {
        v.rest = 2 * rows;
        v.total = v.rest + paged_layout(h, T, max_ctx).total;
        return v;
    }
    v.split = h.fast_attn && T < h.n_cu;
    v.seq = 2 * rows;
    v.ctx = 3 * rows;
    v.budget = 4 * rows;
    v.idx = 5 * rows;
    v.attn = v.idx + align_up((size_t)T * (size_t)h.cfg.max_topk * sizeof(int32_t));
    v.rest = v.attn + align_up(v.split ? sa::attention_workspace(h, T, true) : 0);
    v.total = v.rest + align_up(sa::prefill_varlen_workspace(h, T, (int32_t)max_ctx));
    return v;
}

}  // namespace

namespace sa {

KernelTimer::KernelTimer(sa_handle_s &h, int kind, hipStream_t st) : h_(h), kind_(kind), st_(st)
{
    if (!h_.profiling) return;
    if (h_.spare_events.empty()) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        h_.spare_events.push_back(e);
    }
    start_ = h_.spare_events.back();
    h_.spare_events.pop_back();
    if (hipEventRecord(start_, st_) != hipSuccess) {
        h_.spare_events.push_back(start_);
        start_ = nullptr;
    }
}

KernelTimer::~KernelTimer()
{
    if (!start_) return;
    hipEvent_t stop;
    if (h_.spare_events.empty()) {
        if (hipEventCreate(&stop) != hipSuccess) {
            h_.spare_events.push_back(start_);
            return;
        }
    } else {
        stop = h_.spare_events.back();
        h_.spare_events.pop_back();
    }
    (void)hipEventRecord(stop, st_);
    h_.pending[kind_].emplace_back(start_, stop);
    size_t n = 0;
    for (int k = 0; k < SA_KERNEL_COUNT; ++k) n += h_.pending[k].size();
    if (n >= 2048) (void)drain_profile(h_);
}

hipError_t drain_profile(sa_handle_s &h)
{
    hipError_t first = hipSuccess;
    for (int k = 0; k < SA_KERNEL_COUNT; ++k) {
        for (auto &pr : h.pending[k]) {
            float ms = 0.f;
            hipError_t e = hipEventSynchronize(pr.second);
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
            if (e == hipSuccess) {
                h.total_ms[k] += ms;
                h.launches[k] += 1;
            } else if (first == hipSuccess) {
                first = e;
            }
            h.spare_events.push_back(pr.first);
            h.spare_events.push_back(pr.second);
        }
        h.pending[k].clear();
    }
    return first;
}

}  // namespace sa

extern "C" {

}  // extern "C"

namespace {

// The configuration checks and the host half of a handle (kernels picked, nothing on a device yet).
sa_status_t new_handle(const sa_config_t *cfg, sa_handle_t *out, sa_handle_s **made)
{
    g_create_error.clear();
    *made = nullptr;
    if (!cfg || !out) return fail(nullptr, SA_ERR_INVALID_ARG, "cfg and out must not be NULL");
    *out = nullptr;
    const sa_config_t &c = *cfg;
    if (c.dtype != SA_F32 && c.dtype != SA_BF16)
        return fail(nullptr, SA_ERR_INVALID_ARG, "dtype must be SA_F32 or SA_BF16");
    if (c.n_idx_heads < 1 || c.d_idx < 1 || c.n_heads < 1 || c.n_kv_heads < 1 || c.d_qk < 1 || c.d_v < 1)
        return fail(nullptr, SA_ERR_INVALID_ARG, "head counts and widths must be >= 1");
    if (c.n_heads % c.n_kv_heads != 0)
        return fail(nullptr, SA_ERR_INVALID_ARG, "n_heads (%d) must be a multiple of n_kv_heads (%d)",
                    c.n_heads, c.n_kv_heads);
    if (c.v_from_k != 0 && c.v_from_k != 1) return fail(nullptr, SA_ERR_INVALID_ARG, "v_from_k must be 0 or 1");
    if (c.v_from_k && c.d_v > c.d_qk)
        return fail(nullptr, SA_ERR_INVALID_ARG, "v_from_k needs d_v (%d) <= d_qk (%d)", c.d_v, c.d_qk);
    if (c.max_topk < 1 || c.max_topk > kMaxTopk)
        return fail(nullptr, SA_ERR_INVALID_ARG, "max_topk must be in [1, %d]", kMaxTopk);
    if (c.page_size < 1) return fail(nullptr, SA_ERR_INVALID_ARG, "page_size must be >= 1");
    if (!(c.softmax_scale >= 0.f) || !std::isfinite(c.softmax_scale))
        return fail(nullptr, SA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");

    sa_handle_s *h = new (std::nothrow) sa_handle_s();
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "out of host memory");
    h->cfg = c;
    h->scale = c.softmax_scale > 0.f ? c.softmax_scale : (float)(1.0 / std::sqrt((double)c.d_qk));
    h->fast_indexer = c.dtype == SA_BF16 && c.n_idx_heads == 64 && c.d_idx == 128;
    h->fast_decode = h->fast_indexer && c.page_size == 64;
    h->fast_attn = c.dtype == SA_BF16 && c.n_heads == 16 && c.n_kv_heads == 1 && c.d_qk == 576 &&
                   c.d_v == 512 && c.v_from_k == 1;
    if (!h->fast_indexer && (size_t)(c.n_idx_heads * c.d_idx + c.n_idx_heads) * 4 > 64 * 1024) {
        delete h;
        return fail(nullptr, SA_ERR_UNSUPPORTED, "n_idx_heads * d_idx too large for the generic indexer");
    }
    if (!h->fast_attn && (size_t)(c.d_qk + c.max_topk) * 4 > 64 * 1024) {
        delete h;
        return fail(nullptr, SA_ERR_UNSUPPORTED, "d_qk + max_topk too large for the generic attention");
    }
    *made = h;
    return SA_OK;
}

}  // namespace

extern "C" {

sa_status_t sparse_attn_create(const sa_config_t *cfg, sa_handle_t *out)
{
    sa_handle_s *h = nullptr;
    const sa_status_t sv = new_handle(cfg, out, &h);
    if (sv != SA_OK) return sv;
    if (hipGetDevice(&h->device) != hipSuccess ||
        hipDeviceGetAttribute(&h->n_cu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess ||
        h->n_cu < 1) {
        delete h;
        return fail(nullptr, SA_ERR_HIP, "hipGetDevice failed (no HIP device?)");
    }
    if (h->device < 0 || h->device >= kMaxDevices) {
        delete h;
        return fail(nullptr, SA_ERR_UNSUPPORTED, "device ordinal %d beyond the library's %d", h->device, kMaxDevices);
    }
    {
        // the allocation-free decode's array on this device (the current one): its address, once
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch[h->device]) {
            void *ptr = nullptr;
            const hipError_t es = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (es != hipSuccess || !ptr) {
                delete h;
                return fail(nullptr, SA_ERR_HIP, "looking up the device scratch array: %s", hipGetErrorString(es));
            }
            g_scratch[h->device] = ptr;
        }
    }
    hipError_t e = hipMalloc(reinterpret_cast<void **>(&h->d_err), sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(h->d_err, 0, sizeof(uint32_t));
    if (e != hipSuccess) {
        if (h->d_err) (void)hipFree(h->d_err);
        delete h;
        return fail(nullptr, SA_ERR_HIP, "allocating the device error word: %s", hipGetErrorString(e));
    }
    *out = h;
    return SA_OK;
}

sa_status_t sparse_attn_create_host(const sa_config_t *cfg, int32_t n_cu, sa_handle_t *out)
{
    sa_handle_s *h = nullptr;
    if (n_cu < 1 || n_cu > 65535) {
        g_create_error.clear();
        if (out) *out = nullptr;
        return fail(nullptr, SA_ERR_INVALID_ARG, "n_cu must be in [1, 65535]");
    }
    const sa_status_t sv = new_handle(cfg, out, &h);
    if (sv != SA_OK) return sv;
    h->device = -1;  // no device: every launching call stops after its host validation
    h->n_cu = n_cu;
    h->d_err = nullptr;
    *out = h;
    return SA_OK;
}

void sparse_attn_destroy(sa_handle_t h)
{
    if (!h) return;
    if (h->device >= 0) {
        (void)hipDeviceSynchronize();
        (void)sa::drain_profile(*h);
        for (hipEvent_t e : h->spare_events) (void)hipEventDestroy(e);
        sa::destroy_projection_state(*h);
        (void)hipFree(h->d_err);
    }
    delete h;
}

sa_status_t sparse_attn_profile(sa_handle_t h, int enable)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    sa_status_t s = hip_status(h, sa::drain_profile(*h), "draining timing events");
    for (int k = 0; k < SA_KERNEL_COUNT; ++k) {
        h->total_ms[k] = 0.0;
        h->launches[k] = 0;
    }
    h->profiling = enable != 0;
    return s;
}

sa_status_t sparse_attn_profile_read(sa_handle_t h, double *total_ms, int64_t *launches)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    if (!total_ms || !launches) return fail(h, SA_ERR_INVALID_ARG, "NULL output array");
    sa_status_t s = hip_status(h, sa::drain_profile(*h), "reading timing events");
    for (int k = 0; k < SA_KERNEL_COUNT; ++k) {
        total_ms[k] = h->total_ms[k];
        launches[k] = h->launches[k];
    }
    return s;
}

const char *sparse_attn_last_error(sa_handle_t h)
{
    return h ? h->last_error.c_str() : g_create_error.c_str();
}

sa_status_t sparse_attn_workspace_size(sa_handle_t h, int op, int64_t n, int64_t max_ctx, size_t *bytes)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    if (!bytes) return fail(h, SA_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    if (n < 1) return fail(h, SA_ERR_INVALID_ARG, "n must be >= 1");
    switch (op) {
    case SA_OP_PREFILL:
    case SA_OP_PREFILL_BLOCKS:
        if (n > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "L exceeds int32 token indices");
        *bytes = prefill_layout(*h, n, op == SA_OP_PREFILL_BLOCKS).total;
        if (op == SA_OP_PREFILL_BLOCKS && h->fast_indexer) {
            // the block size is not known here: room for either two-tier path
            const size_t fused = blocks_fused_layout(*h, n).total;
            if (fused > *bytes) *bytes = fused;
        }
        return SA_OK;
    case SA_OP_DECODE:
    case SA_OP_DECODE_BLOCKS:
        if (max_ctx < 1 || max_ctx > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "max_ctx must be in [1, 2^31)");
        *bytes = decode_layout(*h, n, max_ctx).total;
        return SA_OK;
    case SA_OP_PREFILL_CHUNK:
        if (n > INT32_MAX || max_ctx < n || max_ctx > INT32_MAX)
            return fail(h, SA_ERR_INVALID_ARG, "need 1 <= C <= pos0 + C = max_ctx < 2^31");
        *bytes = chunk_layout(*h, max_ctx - n, n).total;
        return SA_OK;
    case SA_OP_PREFILL_PAGED:
        if (n > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "T exceeds the launch limit");
        if (max_ctx < 1 || max_ctx > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "max_ctx must be in [1, 2^31)");
        *bytes = paged_layout(*h, n, max_ctx).total;
        return SA_OK;
    case SA_OP_PREFILL_VARLEN:
        if (n > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "T exceeds the launch limit");
        if (max_ctx < 1 || max_ctx > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "max_ctx must be in [1, 2^31)");
        *bytes = varlen_api_layout(*h, n, max_ctx).total;
        return SA_OK;
    case SA_OP_TOPK:
        *bytes = 0;
        return SA_OK;
    case SA_OP_PROJECT:
        *bytes = sa::projection_workspace();
        return SA_OK;
    case SA_OP_ACCEPT:
        if (max_ctx < 1) return fail(h, SA_ERR_INVALID_ARG, "V must be >= 1");
        *bytes = sa::acceptance_workspace(*h, n, max_ctx);
        return SA_OK;
    default:
        return fail(h, SA_ERR_INVALID_ARG, "unknown op %d", op);
    }
}

sa_status_t sparse_attn_check(sa_handle_t h, void *stream, uint32_t *bits)
{
    if (bits) *bits = 0;
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    if (h->device < 0) return check_device(h);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    sa_status_t s = hip_status(h, hipStreamSynchronize(st), "hipStreamSynchronize");
    if (s != SA_OK) return s;
    uint32_t v = 0;
    s = hip_status(h, hipMemcpy(&v, h->d_err, sizeof(v), hipMemcpyDeviceToHost), "reading the error word");
    if (s != SA_OK) return s;
    if (bits) *bits = v;
    if (v == 0) return SA_OK;
    s = hip_status(h, hipMemset(h->d_err, 0, sizeof(uint32_t)), "clearing the error word");
    if (s != SA_OK) return s;
    return fail(h, SA_ERR_DEVICE_CHECK, "device-side check failed, bits 0x%x", v);
}

sa_status_t indexer_scores(sa_handle_t h, const void *q_idx, const float *w, const void *k_idx,
                           int64_t L, float *scores, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (!q_idx || !w || !k_idx || !scores) return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (L < 1) return fail(h, SA_ERR_INVALID_ARG, "L must be >= 1");
    if (L > kMaxIndexerScoresL)
        return fail(h, SA_ERR_UNSUPPORTED, "indexer_scores materialises [L, L]; L must be <= %lld",
                    (long long)kMaxIndexerScoresL);
    if (!aligned16(q_idx) || !aligned16(k_idx)) return fail(h, SA_ERR_INVALID_ARG, "q_idx/k_idx must be 16-byte aligned");
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    sa::RowSource keys{k_idx, h->cfg.d_idx, nullptr, 0, 0, 0};
    sa::Visibility vis{0, nullptr, 0};
    return hip_status(h, sa::launch_indexer(*h, q_idx, w, L, keys, vis, scores, L, L,
                                            reinterpret_cast<hipStream_t>(stream)),
                      "indexer launch");
}

sa_status_t topk_select(sa_handle_t h, const float *scores, int64_t rows, int64_t cols, int64_t ld,
                        const int32_t *valid_len, const int32_t *k_per_row, int32_t k, int32_t *idx,
                        void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (!scores || !idx) return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (rows < 1 || cols < 1) return fail(h, SA_ERR_INVALID_ARG, "rows and cols must be >= 1");
    if (cols > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "cols exceeds int32 indices");
    if (rows > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "rows exceeds the launch limit");
    if (ld < cols) return fail(h, SA_ERR_INVALID_ARG, "ld (%lld) < cols (%lld)", (long long)ld, (long long)cols);
    if (k < 1 || k > h->cfg.max_topk)
        return fail(h, SA_ERR_INVALID_ARG, "k (%d) must be in [1, max_topk=%d]", k, h->cfg.max_topk);
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    return hip_status(h, sa::launch_topk(*h, scores, ld, rows, cols, valid_len, 0, k_per_row, k, idx, k,
                                         h->d_err, reinterpret_cast<hipStream_t>(stream)),
                      "top-k launch");
}

sa_status_t topk_select_blocks(sa_handle_t h, const float *scores, int64_t rows, int64_t cols, int64_t ld,
                               const int32_t *valid_len, const int32_t *k_per_row, int32_t k, int32_t block_size,
                               int32_t n_blocks, int32_t *idx, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (!scores || !idx) return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (rows < 1 || cols < 1) return fail(h, SA_ERR_INVALID_ARG, "rows and cols must be >= 1");
    if (cols > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "cols exceeds int32 indices");
    if (rows > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "rows exceeds the launch limit");
    if (ld < cols) return fail(h, SA_ERR_INVALID_ARG, "ld (%lld) < cols (%lld)", (long long)ld, (long long)cols);
    if (k < 1 || k > h->cfg.max_topk)
        return fail(h, SA_ERR_INVALID_ARG, "k (%d) must be in [1, max_topk=%d]", k, h->cfg.max_topk);
    sa_status_t s = check_block_select(h, BlockSelect{block_size, n_blocks}, cols);
    if (s != SA_OK) return s;
    s = check_device(h);
    if (s != SA_OK) return s;
    return hip_status(h, sa::launch_block_topk(*h, scores, ld, rows, cols, valid_len, 0, k_per_row, k, block_size,
                                               n_blocks, nullptr, 0, idx, k, h->d_err,
                                               reinterpret_cast<hipStream_t>(stream)),
                      "block top-k launch");
}

sa_status_t sparse_attn_prefill(sa_handle_t h, const void *q, const void *k, const void *v,
                                const void *q_idx, const float *w, const void *k_idx, int64_t L,
                                int32_t topk, float *out, float *lse, int32_t *idx_out, void *ws,
                                size_t ws_bytes, void *stream)
{
    return prefill_impl(h, q, k, v, q_idx, w, k_idx, L, topk, nullptr, out, lse, idx_out, ws, ws_bytes, stream);
}

sa_status_t sparse_attn_prefill_blocks(sa_handle_t h, const void *q, const void *k, const void *v,
                                       const void *q_idx, const float *w, const void *k_idx, int64_t L,
                                       int32_t topk, int32_t block_size, int32_t n_blocks, float *out, float *lse,
                                       int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    const BlockSelect b{block_size, n_blocks};
    return prefill_impl(h, q, k, v, q_idx, w, k_idx, L, topk, &b, out, lse, idx_out, ws, ws_bytes, stream);
}

sa_status_t sparse_attn_decode(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                               const void *kv_pages, const void *v_pages, const void *kidx_pages,
                               int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                               const int32_t *ctx_len, const int32_t *topk, int32_t B, int32_t max_ctx,
                               float *out, float *lse, int32_t *idx_out, void *ws, size_t ws_bytes,
                               void *stream)
{
    return decode_impl(h, q, q_idx, w, kv_pages, v_pages, kidx_pages, n_pages, block_table, max_blocks, ctx_len,
                       topk, B, max_ctx, nullptr, out, lse, idx_out, ws, ws_bytes, stream);
}

sa_status_t sparse_attn_decode_blocks(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                      const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                      const int32_t *ctx_len, const int32_t *topk, int32_t B, int32_t max_ctx,
                                      int32_t block_size, int32_t n_blocks, float *out, float *lse,
                                      int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    const BlockSelect b{block_size, n_blocks};
    return decode_impl(h, q, q_idx, w, kv_pages, v_pages, kidx_pages, n_pages, block_table, max_blocks, ctx_len,
                       topk, B, max_ctx, &b, out, lse, idx_out, ws, ws_bytes, stream);
}

sa_status_t sparse_attn_decode_noalloc(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                       const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                       int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                                       const int32_t *ctx_len, const int32_t *topk, int32_t B, int32_t max_ctx,
                                       float *out, float *lse, int32_t *idx_out, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (B < 1 || B > 65535) return fail(h, SA_ERR_INVALID_ARG, "B must be in [1, 65535]");
    if (max_ctx < 1) return fail(h, SA_ERR_INVALID_ARG, "max_ctx must be >= 1");
    const size_t need = decode_layout(*h, B, max_ctx).total;
    if (need > kNoAllocBytes)
        return fail(h, SA_ERR_UNSUPPORTED,
                    "the allocation-free decode holds %zu bytes of device scratch; B = %d, max_ctx = %d, max_topk = %d "
                    "need %zu (use sparse_attn_decode with a workspace)",
                    kNoAllocBytes, B, max_ctx, h->cfg.max_topk, need);
    if (h->device < 0) return check_device(h);
    void *ptr = g_scratch[h->device];  // set when the handle was created on this device
    return decode_impl(h, q, q_idx, w, kv_pages, v_pages, kidx_pages, n_pages, block_table, max_blocks, ctx_len,
                       topk, B, max_ctx, nullptr, out, lse, idx_out, ptr, kNoAllocBytes, stream);
}

}  // extern "C"

namespace {

sa_status_t prefill_impl(sa_handle_t h, const void *q, const void *k, const void *v, const void *q_idx,
                         const float *w, const void *k_idx, int64_t L, int32_t topk, const BlockSelect *blocks,
                         float *out, float *lse, int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    const sa_config_t &c = h->cfg;
    if (!q || !k || !q_idx || !w || !k_idx || !out) return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (c.v_from_k ? v != nullptr : v == nullptr)
        return fail(h, SA_ERR_INVALID_ARG, c.v_from_k ? "v must be NULL when v_from_k = 1"
                                                      : "v must not be NULL when v_from_k = 0");
    if (L < 1 || L > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "L must be in [1, 2^31)");
    if (topk < 1 || topk > c.max_topk)
        return fail(h, SA_ERR_INVALID_ARG, "topk (%d) must be in [1, max_topk=%d]", topk, c.max_topk);
    if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || !aligned16(q_idx) || !aligned16(k_idx) ||
        !aligned16(w) || !aligned16(out))
        return fail(h, SA_ERR_INVALID_ARG, "q, k, v, q_idx, w, k_idx and out must be 16-byte aligned");
    if (blocks) {
        const sa_status_t sb = check_block_select(h, *blocks, L);
        if (sb != SA_OK) return sb;
    }
    const bool fused_blocks = blocks && blocks_fused(*h, blocks->block_size);
    const PrefillLayout lay = prefill_layout(*h, L, blocks != nullptr);
    const size_t need = fused_blocks ? blocks_fused_layout(*h, L).total : lay.total;
    if (!ws || ws_bytes < need)
        return fail(h, SA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *base = reinterpret_cast<char *>(ws);
    if (fused_blocks) {
        // the fused indexer writes each row's best score per 64-key tile; the kept blocks' tokens are then
        // scored again (bit-identical scores) and selected per row
        const BlocksFusedLayout bl = blocks_fused_layout(*h, L);
        int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + bl.idx);
        uint32_t *keys = reinterpret_cast<uint32_t *>(base + bl.keys);
        s = hip_status(h, sa::launch_prefill_topk(*h, q_idx, w, k_idx, L, topk, idx, base + bl.counter, st, nullptr, 0,
                                                  0, keys, (int64_t)blocks->n_blocks * blocks->block_size),
                       "block-key launch");
        if (s != SA_OK) return s;
        s = hip_status(h, sa::launch_block_rescore_topk(*h, q_idx, w, k_idx, nullptr, 0, L, 0, topk, blocks->block_size,
                                                        blocks->n_blocks, keys, (int64_t)sa::prefill_block_keys_ld(L, 0),
                                                        idx, st),
                       "block rescore launch");
        if (s != SA_OK) return s;
        sa::RowSource kv{k, (int64_t)c.n_kv_heads * c.d_qk, nullptr, 0, 0, 0};
        sa::RowSource vv{v, (int64_t)c.n_kv_heads * c.d_v, nullptr, 0, 0, 0};
        sa::Visibility vis{0, nullptr, 0};
        sa::Selection sel{idx, topk, topk, nullptr};
        return hip_status(h, sa::launch_attention(*h, q, L, kv, vv, vis, sel, out, lse, nullptr, st),
                          "attention launch");
    }
    float *scores = reinterpret_cast<float *>(base + lay.scores);
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + lay.idx);
    const size_t es = elem_size(*h);

    if (h->fast_indexer && !blocks) {
        // fused indexer + streaming top-k: no score matrix at all
        s = hip_status(h, sa::launch_prefill_topk(*h, q_idx, w, k_idx, L, topk, idx, base + lay.scores, st),
                       "indexer/top-k launch");
        if (s != SA_OK) return s;
    } else {
        // indexer -> top-k per block of query rows; the block's scores live in the workspace
        const int64_t chunk = prefill_chunk_rows(L);
        sa::RowSource keys{k_idx, c.d_idx, nullptr, 0, 0, 0};
        for (int64_t r0 = 0; r0 < L; r0 += chunk) {
            const int64_t rows = r0 + chunk < L ? chunk : L - r0;
            const int64_t cols = r0 + rows;  // keys any row of the block can see
            sa::Visibility vis{r0, nullptr, 0};
            s = hip_status(h, sa::launch_indexer(*h, reinterpret_cast<const char *>(q_idx) + r0 * c.n_idx_heads * c.d_idx * es,
                                                 w + r0 * c.n_idx_heads, rows, keys, vis, scores, cols, cols, st),
                           "indexer launch");
            if (s != SA_OK) return s;
            if (blocks)
                s = hip_status(h, sa::launch_block_topk(*h, scores, cols, rows, cols, nullptr, r0, nullptr, topk,
                                                        blocks->block_size, blocks->n_blocks, nullptr, 0,
                                                        idx + r0 * topk, topk, h->d_err, st),
                               "block top-k launch");
            else
                s = hip_status(h, sa::launch_topk(*h, scores, cols, rows, cols, nullptr, r0, nullptr, topk,
                                                  idx + r0 * topk, topk, h->d_err, st),
                               "top-k launch");
            if (s != SA_OK) return s;
        }
    }
    sa::RowSource kv{k, (int64_t)c.n_kv_heads * c.d_qk, nullptr, 0, 0, 0};
    sa::RowSource vv{v, (int64_t)c.n_kv_heads * c.d_v, nullptr, 0, 0, 0};
    sa::Visibility vis{0, nullptr, 0};
    sa::Selection sel{idx, topk, topk, nullptr};
    return hip_status(h, sa::launch_attention(*h, q, L, kv, vv, vis, sel, out, lse, nullptr, st),
                      "attention launch");
}

sa_status_t decode_impl(sa_handle_t h, const void *q, const void *q_idx, const float *w, const void *kv_pages,
                        const void *v_pages, const void *kidx_pages, int64_t n_pages, const int32_t *block_table,
                        int32_t max_blocks, const int32_t *ctx_len, const int32_t *topk, int32_t B, int32_t max_ctx,
                        const BlockSelect *blocks, float *out, float *lse, int32_t *idx_out, void *ws,
                        size_t ws_bytes, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    const sa_config_t &c = h->cfg;
    if (!q || !q_idx || !w || !kv_pages || !kidx_pages || !block_table || !ctx_len || !topk || !out)
        return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (c.v_from_k ? v_pages != nullptr : v_pages == nullptr)
        return fail(h, SA_ERR_INVALID_ARG, c.v_from_k ? "v_pages must be NULL when v_from_k = 1"
                                                      : "v_pages must not be NULL when v_from_k = 0");
    if (B < 1 || B > 65535) return fail(h, SA_ERR_INVALID_ARG, "B must be in [1, 65535]");
    if (n_pages < 1) return fail(h, SA_ERR_INVALID_ARG, "n_pages must be >= 1");
    if (max_blocks < 1) return fail(h, SA_ERR_INVALID_ARG, "max_blocks must be >= 1");
    if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)max_blocks * c.page_size)
        return fail(h, SA_ERR_INVALID_ARG, "max_ctx (%d) must be in [1, max_blocks * page_size = %lld]",
                    max_ctx, (long long)max_blocks * c.page_size);
    if (!aligned16(q) || !aligned16(q_idx) || !aligned16(kv_pages) || !aligned16(kidx_pages) ||
        (v_pages && !aligned16(v_pages)) || !aligned16(w) || !aligned16(out))
        return fail(h, SA_ERR_INVALID_ARG, "q, q_idx, w, out and the page pools must be 16-byte aligned");
    if (blocks) {
        const sa_status_t sb = check_block_select(h, *blocks, max_ctx);
        if (sb != SA_OK) return sb;
    }
    const DecodeLayout lay = decode_layout(*h, B, max_ctx);
    if (!ws || ws_bytes < lay.total)
        return fail(h, SA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total, ws_bytes);
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *base = reinterpret_cast<char *>(ws);
    float *scores = reinterpret_cast<float *>(base + lay.scores);
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + lay.idx);

    sa::Visibility vis{0, ctx_len, max_ctx};
    if (blocks) {
        // scores of every cached token, then the two-tier selection per sequence
        int64_t ld = max_ctx, pmax_ld = 0;
        const uint32_t *pmax = nullptr;
        if (h->fast_decode) {
            const sa::DecodeTopkLayout dl = sa::decode_topk_layout(B, max_ctx);
            const bool use_pmax = blocks->block_size >= 64;
            s = hip_status(h, sa::launch_decode_indexer(*h, q_idx, w, kidx_pages, n_pages, block_table, max_blocks,
                                                        ctx_len, nullptr, B, max_ctx, use_pmax, base + lay.scores,
                                                        st),
                           "decode indexer launch");
            scores = reinterpret_cast<float *>(base + lay.scores + dl.scores);
            ld = dl.ld;
            if (use_pmax) {
                pmax = reinterpret_cast<const uint32_t *>(base + lay.scores + dl.pmax);
                pmax_ld = dl.pmax_ld;
            }
        } else {
            sa::RowSource keys{kidx_pages, c.d_idx, block_table, max_blocks, c.page_size, n_pages};
            s = hip_status(h, sa::launch_indexer(*h, q_idx, w, B, keys, vis, scores, max_ctx, max_ctx, st),
                           "indexer launch");
        }
        if (s != SA_OK) return s;
        s = hip_status(h, sa::launch_block_topk(*h, scores, ld, B, max_ctx, ctx_len, 0, topk, c.max_topk,
                                                blocks->block_size, blocks->n_blocks, pmax, pmax_ld, idx, c.max_topk,
                                                h->d_err, st),
                       "block top-k launch");
        if (s != SA_OK) return s;
    } else if (h->fast_decode) {
        s = hip_status(h, sa::launch_decode_indexer_topk(*h, q_idx, w, kidx_pages, n_pages, block_table, max_blocks,
                                                         ctx_len, topk, B, max_ctx, idx, base + lay.scores, st),
                       "decode indexer/top-k launch");
        if (s != SA_OK) return s;
    } else {
        sa::RowSource keys{kidx_pages, c.d_idx, block_table, max_blocks, c.page_size, n_pages};
        s = hip_status(h, sa::launch_indexer(*h, q_idx, w, B, keys, vis, scores, max_ctx, max_ctx, st),
                       "indexer launch");
        if (s != SA_OK) return s;
        s = hip_status(h, sa::launch_topk(*h, scores, max_ctx, B, max_ctx, ctx_len, 0, topk, c.max_topk, idx,
                                          c.max_topk, h->d_err, st),
                       "top-k launch");
        if (s != SA_OK) return s;
    }
    sa::RowSource kv{kv_pages, (int64_t)c.n_kv_heads * c.d_qk, block_table, max_blocks, c.page_size, n_pages};
    sa::RowSource vv{v_pages, (int64_t)c.n_kv_heads * c.d_v, block_table, max_blocks, c.page_size, n_pages};
    sa::Selection sel{idx, c.max_topk, c.max_topk, topk};
    return hip_status(h, sa::launch_attention(*h, q, B, kv, vv, vis, sel, out, lse, base + lay.attn, st),
                      "attention launch");
}

}  // namespace

extern "C" {

sa_status_t sparse_attn_prefill_paged(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                      const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table, int32_t n_seqs,
                                      int32_t max_blocks, const int32_t *row_seq, const int32_t *row_pos,
                                      int64_t T, int32_t max_ctx, int32_t topk, float *out, float *lse,
                                      int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    const sa_config_t &c = h->cfg;
    if (!q || !q_idx || !w || !kv_pages || !kidx_pages || !block_table || !row_seq || !row_pos || !out)
        return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (c.v_from_k ? v_pages != nullptr : v_pages == nullptr)
        return fail(h, SA_ERR_INVALID_ARG, c.v_from_k ? "v_pages must be NULL when v_from_k = 1"
                                                      : "v_pages must not be NULL when v_from_k = 0");
    if (T < 1 || T > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "T must be in [1, 2^31)");
    if (n_seqs < 1) return fail(h, SA_ERR_INVALID_ARG, "n_seqs must be >= 1");
    if (n_pages < 1) return fail(h, SA_ERR_INVALID_ARG, "n_pages must be >= 1");
    if (max_blocks < 1) return fail(h, SA_ERR_INVALID_ARG, "max_blocks must be >= 1");
    if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)max_blocks * c.page_size)
        return fail(h, SA_ERR_INVALID_ARG, "max_ctx (%d) must be in [1, max_blocks * page_size = %lld]",
                    max_ctx, (long long)max_blocks * c.page_size);
    if (topk < 1 || topk > c.max_topk)
        return fail(h, SA_ERR_INVALID_ARG, "topk (%d) must be in [1, max_topk=%d]", topk, c.max_topk);
    if (!aligned16(q) || !aligned16(q_idx) || !aligned16(kv_pages) || !aligned16(kidx_pages) ||
        (v_pages && !aligned16(v_pages)) || !aligned16(w) || !aligned16(out))
        return fail(h, SA_ERR_INVALID_ARG, "q, q_idx, w, out and the page pools must be 16-byte aligned");
    const PagedLayout lay = paged_layout(*h, T, max_ctx);
    if (!ws || ws_bytes < lay.total)
        return fail(h, SA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total, ws_bytes);
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *base = reinterpret_cast<char *>(ws);
    int32_t *seq = reinterpret_cast<int32_t *>(base + lay.seq);
    int32_t *ctx = reinterpret_cast<int32_t *>(base + lay.ctx);
    int32_t *budget = reinterpret_cast<int32_t *>(base + lay.budget);
    float *scores = reinterpret_cast<float *>(base + lay.scores);
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + lay.idx);
    const size_t es = elem_size(*h);

    s = hip_status(h, sa::launch_paged_rows(*h, row_seq, row_pos, T, n_seqs, max_ctx, topk, seq, ctx, budget, st),
                   "row check launch");
    if (s != SA_OK) return s;
    if (lay.fused) {
        // rows sorted by (sequence, position) on the device, each sequence's run in tiles of 8 rows sharing
        // every key tile (one page)
        s = hip_status(h, sa::launch_prefill_rows(*h, q_idx, w, kidx_pages, n_pages, block_table, max_blocks, row_seq,
                                                  row_pos, n_seqs, T, max_ctx, topk, idx, base + lay.scores, st),
                       "row-tile indexer/top-k launch");
        if (s != SA_OK) return s;
    }
    // otherwise indexer -> top-k per block of query rows, each row over its own sequence's pages
    for (int64_t r0 = 0; !lay.fused && r0 < T; r0 += lay.chunk) {
        const int32_t rows = (int32_t)(r0 + lay.chunk < T ? lay.chunk : T - r0);
        const void *qi = reinterpret_cast<const char *>(q_idx) + r0 * c.n_idx_heads * c.d_idx * es;
        const float *wr = w + r0 * c.n_idx_heads;
        if (h->fast_decode) {
            s = hip_status(h, sa::launch_decode_indexer(*h, qi, wr, kidx_pages, n_pages, block_table, max_blocks,
                                                        ctx + r0, seq + r0, rows, max_ctx, false, scores, st),
                           "decode indexer launch");
            if (s != SA_OK) return s;
            s = hip_status(h, sa::launch_decode_topk(*h, ctx + r0, budget + r0, topk, rows, max_ctx, idx + r0 * topk,
                                                     scores, st),
                           "top-k launch");
        } else {
            sa::RowSource keys{kidx_pages, c.d_idx, block_table, max_blocks, c.page_size, n_pages, seq + r0};
            sa::Visibility vis{0, ctx + r0, max_ctx};
            s = hip_status(h, sa::launch_indexer(*h, qi, wr, rows, keys, vis, scores, max_ctx, max_ctx, st),
                           "indexer launch");
            if (s != SA_OK) return s;
            s = hip_status(h, sa::launch_topk(*h, scores, max_ctx, rows, max_ctx, ctx + r0, 0, nullptr, topk,
                                              idx + r0 * topk, topk, h->d_err, st),
                           "top-k launch");
        }
        if (s != SA_OK) return s;
    }
    sa::RowSource kv{kv_pages, (int64_t)c.n_kv_heads * c.d_qk, block_table, max_blocks, c.page_size, n_pages, seq};
    sa::RowSource vv{v_pages, (int64_t)c.n_kv_heads * c.d_v, block_table, max_blocks, c.page_size, n_pages, seq};
    sa::Visibility vis{0, ctx, max_ctx};
    sa::Selection sel{idx, topk, topk, nullptr};
    return hip_status(h, sa::launch_attention(*h, q, T, kv, vv, vis, sel, out, lse, base + lay.attn, st, lay.split),
                      "attention launch");
}

sa_status_t sparse_attn_prefill_varlen(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                       const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                       int64_t n_pages, const int32_t *block_table, int32_t n_seqs,
                                       int32_t max_blocks, const int32_t *cu_seqlens, const int32_t *ctx_len,
                                       int64_t T, int32_t max_ctx, int32_t topk, float *out, float *lse,
                                       int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    const sa_config_t &c = h->cfg;
    if (!q || !q_idx || !w || !kv_pages || !kidx_pages || !block_table || !cu_seqlens || !ctx_len || !out)
        return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (c.v_from_k ? v_pages != nullptr : v_pages == nullptr)
        return fail(h, SA_ERR_INVALID_ARG, c.v_from_k ? "v_pages must be NULL when v_from_k = 1"
                                                      : "v_pages must not be NULL when v_from_k = 0");
    if (T < 1 || T > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "T must be in [1, 2^31)");
    if (n_seqs < 1) return fail(h, SA_ERR_INVALID_ARG, "n_seqs must be >= 1");
    if (n_pages < 1) return fail(h, SA_ERR_INVALID_ARG, "n_pages must be >= 1");
    if (max_blocks < 1) return fail(h, SA_ERR_INVALID_ARG, "max_blocks must be >= 1");
    if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)max_blocks * c.page_size)
        return fail(h, SA_ERR_INVALID_ARG, "max_ctx (%d) must be in [1, max_blocks * page_size = %lld]",
                    max_ctx, (long long)max_blocks * c.page_size);
    if (topk < 1 || topk > c.max_topk)
        return fail(h, SA_ERR_INVALID_ARG, "topk (%d) must be in [1, max_topk=%d]", topk, c.max_topk);
    if (!aligned16(q) || !aligned16(q_idx) || !aligned16(kv_pages) || !aligned16(kidx_pages) ||
        (v_pages && !aligned16(v_pages)) || !aligned16(w) || !aligned16(out))
        return fail(h, SA_ERR_INVALID_ARG, "q, q_idx, w, out and the page pools must be 16-byte aligned");
    const VarlenApiLayout lay = varlen_api_layout(*h, T, max_ctx);
    if (!ws || ws_bytes < lay.total)
        return fail(h, SA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total, ws_bytes);
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *base = reinterpret_cast<char *>(ws);
    int32_t *row_seq = reinterpret_cast<int32_t *>(base + lay.row_seq);
    int32_t *row_pos = reinterpret_cast<int32_t *>(base + lay.row_pos);
    if (!varlen_fused(*h, max_ctx)) {
        // the rows' (sequence, position) pairs, then the paged rows' path
        s = hip_status(h, sa::launch_varlen_rows(*h, cu_seqlens, ctx_len, n_seqs, T, max_ctx, topk, nullptr, row_seq,
                                                 row_pos, st),
                       "row layout launch");
        if (s != SA_OK) return s;
        return sparse_attn_prefill_paged(h, q, q_idx, w, kv_pages, v_pages, kidx_pages, n_pages, block_table, n_seqs,
                                         max_blocks, row_seq, row_pos, T, max_ctx, topk, out, lse, idx_out,
                                         base + lay.rest, ws_bytes - lay.rest, stream);
    }
    int32_t *seq = reinterpret_cast<int32_t *>(base + lay.seq);
    int32_t *ctx = reinterpret_cast<int32_t *>(base + lay.ctx);
    int32_t *budget = reinterpret_cast<int32_t *>(base + lay.budget);
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + lay.idx);
    s = hip_status(h, sa::launch_varlen_rows(*h, cu_seqlens, ctx_len, n_seqs, T, max_ctx, topk, idx, row_seq, row_pos,
                                             st),
                   "row layout launch");
    if (s != SA_OK) return s;
    s = hip_status(h, sa::launch_paged_rows(*h, row_seq, row_pos, T, n_seqs, max_ctx, topk, seq, ctx, budget, st),
                   "row check launch");
    if (s != SA_OK) return s;
    s = hip_status(h, sa::launch_prefill_varlen(*h, q_idx, w, kidx_pages, n_pages, block_table, max_blocks,
                                                cu_seqlens, ctx_len, n_seqs, T, max_ctx, topk, idx, base + lay.rest,
                                                st),
                   "indexer/top-k launch");
    if (s != SA_OK) return s;
    sa::RowSource kv{kv_pages, (int64_t)c.n_kv_heads * c.d_qk, block_table, max_blocks, c.page_size, n_pages, seq};
    sa::RowSource vv{v_pages, (int64_t)c.n_kv_heads * c.d_v, block_table, max_blocks, c.page_size, n_pages, seq};
    sa::Visibility vis{0, ctx, max_ctx};
    sa::Selection sel{idx, topk, topk, nullptr};
    return hip_status(h, sa::launch_attention(*h, q, T, kv, vv, vis, sel, out, lse, base + lay.attn, st, lay.split),
                      "attention launch");
}

sa_status_t sparse_attn_prefill_chunk(sa_handle_t h, const void *q, const void *q_idx, const float *w,
                                      const void *kv_pages, const void *v_pages, const void *kidx_pages,
                                      int64_t n_pages, const int32_t *block_table_row, int32_t max_blocks,
                                      int64_t pos0, int64_t C, int32_t topk, float *out, float *lse,
                                      int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    const sa_config_t &c = h->cfg;
    if (!q || !q_idx || !w || !kv_pages || !kidx_pages || !block_table_row || !out)
        return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (c.v_from_k ? v_pages != nullptr : v_pages == nullptr)
        return fail(h, SA_ERR_INVALID_ARG, c.v_from_k ? "v_pages must be NULL when v_from_k = 1"
                                                      : "v_pages must not be NULL when v_from_k = 0");
    if (n_pages < 1) return fail(h, SA_ERR_INVALID_ARG, "n_pages must be >= 1");
    if (max_blocks < 1) return fail(h, SA_ERR_INVALID_ARG, "max_blocks must be >= 1");
    if (pos0 < 0 || C < 1 || pos0 + C > (int64_t)max_blocks * c.page_size || pos0 + C > INT32_MAX)
        return fail(h, SA_ERR_INVALID_ARG, "need pos0 >= 0, C >= 1, pos0 + C <= max_blocks * page_size = %lld",
                    (long long)max_blocks * c.page_size);
    if (topk < 1 || topk > c.max_topk)
        return fail(h, SA_ERR_INVALID_ARG, "topk (%d) must be in [1, max_topk=%d]", topk, c.max_topk);
    if (!aligned16(q) || !aligned16(q_idx) || !aligned16(kv_pages) || !aligned16(kidx_pages) ||
        (v_pages && !aligned16(v_pages)) || !aligned16(w) || !aligned16(out))
        return fail(h, SA_ERR_INVALID_ARG, "q, q_idx, w, out and the page pools must be 16-byte aligned");
    const PrefillLayout lay = chunk_layout(*h, pos0, C);
    if (!ws || ws_bytes < lay.total)
        return fail(h, SA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total, ws_bytes);
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *base = reinterpret_cast<char *>(ws);
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + lay.idx);
    const size_t es = elem_size(*h);
    // every query row reads the one block-table row: a row stride of 0
    sa::RowSource kv{kv_pages, (int64_t)c.n_kv_heads * c.d_qk, block_table_row, 0, c.page_size, n_pages};
    sa::RowSource vv{v_pages, (int64_t)c.n_kv_heads * c.d_v, block_table_row, 0, c.page_size, n_pages};

    if (chunk_fused(*h, pos0, C)) {
        s = hip_status(h, sa::launch_prefill_topk(*h, q_idx, w, kidx_pages, C, topk, idx, base + lay.scores, st,
                                                  block_table_row, n_pages, pos0),
                       "indexer/top-k launch");
        if (s != SA_OK) return s;
    } else {
        float *scores = reinterpret_cast<float *>(base + lay.scores);
        sa::RowSource keys{kidx_pages, c.d_idx, block_table_row, 0, c.page_size, n_pages};
        const int64_t n = pos0 + C;
        int64_t chunk = (int64_t)(kPrefillChunkBytes / (sizeof(float) * (size_t)n));
        chunk = chunk < 1 ? 1 : (chunk > C ? C : chunk);
        if (chunk > 65535) chunk = 65535;
        for (int64_t r0 = 0; r0 < C; r0 += chunk) {
            const int64_t rows = r0 + chunk < C ? chunk : C - r0;
            const int64_t cols = pos0 + r0 + rows;  // keys any row of the block can see
            sa::Visibility vis{pos0 + r0, nullptr, 0};
            s = hip_status(h, sa::launch_indexer(*h, reinterpret_cast<const char *>(q_idx) + r0 * c.n_idx_heads * c.d_idx * es,
                                                 w + r0 * c.n_idx_heads, rows, keys, vis, scores, cols, cols, st),
                           "indexer launch");
            if (s != SA_OK) return s;
            s = hip_status(h, sa::launch_topk(*h, scores, cols, rows, cols, nullptr, pos0 + r0, nullptr, topk,
                                              idx + r0 * topk, topk, h->d_err, st),
                           "top-k launch");
            if (s != SA_OK) return s;
        }
    }
    sa::Visibility vis{pos0, nullptr, 0};
    sa::Selection sel{idx, topk, topk, nullptr};
    return hip_status(h, sa::launch_attention(*h, q, C, kv, vv, vis, sel, out, lse, nullptr, st), "attention launch");
}

sa_status_t acceptance_rate(sa_handle_t h, const float *logits_p, const float *logits_q, int64_t T, int64_t V,
                            int64_t ld, float *alpha, void *ws, size_t ws_bytes, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (!logits_p || !logits_q || !alpha) return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (T < 1 || T > INT32_MAX) return fail(h, SA_ERR_INVALID_ARG, "T must be in [1, 2^31)");
    if (V < 1 || ld < V) return fail(h, SA_ERR_INVALID_ARG, "need 1 <= V <= ld (V %lld, ld %lld)", (long long)V,
                                     (long long)ld);
    if (ws) {
        const size_t need = sa::acceptance_workspace(*h, T, V);
        if (ws_bytes < need)
            return fail(h, SA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
        if (need == 0) ws = nullptr;
    }
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    return hip_status(h, sa::launch_acceptance_rate(*h, logits_p, logits_q, T, V, ld, alpha, ws,
                                                    reinterpret_cast<hipStream_t>(stream)),
                      "acceptance-rate launch");
}

sa_status_t acceptance_bin_stats(sa_handle_t h, const float *alpha, const int32_t *pos, int64_t T, int32_t bin_size,
                                 int32_t n_bins, float percentile, int32_t *count, float *mean, float *pct,
                                 void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (!alpha || !pos || !count || !mean || !pct) return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (T < 1) return fail(h, SA_ERR_INVALID_ARG, "T must be >= 1");
    if (bin_size < 1 || n_bins < 1) return fail(h, SA_ERR_INVALID_ARG, "bin_size and n_bins must be >= 1");
    if (!(percentile >= 0.f && percentile <= 100.f))
        return fail(h, SA_ERR_INVALID_ARG, "percentile must be in [0, 100]");
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    return hip_status(h, sa::launch_bin_stats(*h, alpha, pos, T, bin_size, n_bins, percentile, count, mean, pct,
                                              reinterpret_cast<hipStream_t>(stream)),
                      "bin statistics launch");
}

sa_status_t indexer_project_q(sa_handle_t h, const void *q, int64_t L, const void *W_iq, const void *W_w,
                              void *q_idx, float *w, void *ws, size_t ws_bytes, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (!q) return fail(h, SA_ERR_INVALID_ARG, "q is NULL");
    if (L < 1) return fail(h, SA_ERR_INVALID_ARG, "L must be >= 1");
    if (!W_iq && !W_w) return fail(h, SA_ERR_INVALID_ARG, "nothing to project: W_iq and W_w are both NULL");
    if (!W_iq != !q_idx || !W_w != !w)
        return fail(h, SA_ERR_INVALID_ARG, "W_iq / q_idx and W_w / w must be given (or left NULL) in pairs");
    if (h->cfg.dtype != SA_BF16) return fail(h, SA_ERR_UNSUPPORTED, "the projections take bf16 handles only");
    if (!aligned16(q) || (W_iq && (!aligned16(W_iq) || !aligned16(q_idx))) || (W_w && (!aligned16(W_w) || !aligned16(w))))
        return fail(h, SA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    const int64_t K = (int64_t)h->cfg.n_heads * h->cfg.d_qk, N1 = (int64_t)h->cfg.n_idx_heads * h->cfg.d_idx;
    if (K % 64 != 0 || K > (1 << 24) || N1 % 256 != 0 || h->cfg.n_idx_heads > 256)
        return fail(h, SA_ERR_UNSUPPORTED,
                    "the query projection needs H * d_qk a multiple of 64 up to 2^24 (got %lld), H_I * d_I a "
                    "multiple of 256 (got %lld) and H_I <= 256",
                    (long long)K, (long long)N1);
    (void)ws;  // no workspace is needed
    (void)ws_bytes;
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    return sa::launch_project_q(*h, q, L, W_iq, W_w, q_idx, w, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

sa_status_t indexer_project_k(sa_handle_t h, const void *k, int64_t L, const void *W_ik, void *k_idx,
                              const int32_t *block_table, int32_t n_seqs, int32_t max_blocks, int64_t n_pages,
                              const int32_t *row_seq, const int32_t *row_pos, int64_t pos0, void *stream)
{
    if (!h) return fail(nullptr, SA_ERR_INVALID_ARG, "handle is NULL");
    h->last_error.clear();
    if (!k || !W_ik || !k_idx) return fail(h, SA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (L < 1) return fail(h, SA_ERR_INVALID_ARG, "L must be >= 1");
    const sa_config_t &c = h->cfg;
    if (c.dtype != SA_BF16) return fail(h, SA_ERR_UNSUPPORTED, "the projections take bf16 handles only");
    if (c.d_idx != 128) return fail(h, SA_ERR_UNSUPPORTED, "the key projection needs d_idx = 128 (got %d)", c.d_idx);
    const int kw = c.n_kv_heads * c.d_qk;
    if (kw != 576 && kw != 512 && kw != 256 && kw != 128)
        return fail(h, SA_ERR_UNSUPPORTED, "the key projection serves key rows of 128, 256, 512 or 576 elements (got %d)", kw);
    if (!aligned16(k) || !aligned16(W_ik) || !aligned16(k_idx)) return fail(h, SA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (block_table && (n_seqs < 1 || max_blocks < 1 || n_pages < 1))
        return fail(h, SA_ERR_INVALID_ARG, "a block table needs n_seqs, max_blocks and n_pages >= 1");
    sa_status_t s = check_device(h);
    if (s != SA_OK) return s;
    return hip_status(h, sa::launch_project_k(*h, k, L, W_ik, k_idx, block_table, n_seqs, max_blocks, n_pages, row_seq,
                                              row_pos, pos0, reinterpret_cast<hipStream_t>(stream)),
                      "key projection launch");
}

}  // extern "C"
