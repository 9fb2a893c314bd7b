"""Indexer-selected sparse attention on AMD Instinct MI355X (gfx950).

Python binding of ``libsparse_attn.so`` (declared in ``include/sparse_attn.h``).  The
functions here carry the C names and only marshal arguments: torch tensors become device
pointers, the current HIP stream is passed along, and a non-OK status becomes a
``SparseAttnError``.  Every step of the computation runs in the library's HIP kernels;
there is no Python or CPU fallback, and a missing library raises at import of the first
call.

The method: a lightweight indexer scores every preceding token, I(t,s) = sum_j w(t,j)
ReLU(q(t,j).k(s)) ("Sparse Attention and RL Optimization: Three Technical Breakthroughs in
LLM Post-Training", section 2.2); each query keeps the top-k tokens (section 2.3) and runs
softmax attention over only those KV rows (section 2.5; for decode over a paged cache,
"Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and
Verifiable Synthetic Data", section 2.3).  The ``*_blocks`` variants select with the two-tier
block -> token rule of "A Guide to Sparse Attention and Efficient Reinforcement Learning in
LLM Long-Context Inference", section 1.1.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP, SA_ERR_DEVICE_CHECK = range(6)
SA_F32, SA_BF16 = 0, 1
SA_OP_PREFILL, SA_OP_DECODE, SA_OP_TOPK, SA_OP_PROJECT, SA_OP_PREFILL_BLOCKS, SA_OP_DECODE_BLOCKS = 1, 2, 3, 4, 5, 6
SA_OP_PREFILL_PAGED, SA_OP_PREFILL_CHUNK, SA_OP_PREFILL_VARLEN, SA_OP_ACCEPT = 7, 8, 9, 10
SA_DEVERR_INDEX_RANGE, SA_DEVERR_BLOCK_TABLE, SA_DEVERR_CTX_LEN, SA_DEVERR_TOPK, SA_DEVERR_ROW = 1, 2, 4, 8, 16
SA_DEVERR_SYNC = 32

# Every symbol include/sparse_attn.h declares.
EXPORTED = ("sparse_attn_create", "sparse_attn_create_host", "sparse_attn_destroy", "sparse_attn_last_error",
            "sparse_attn_workspace_size", "sparse_attn_check", "indexer_scores", "topk_select",
            "topk_select_blocks", "sparse_attn_prefill", "sparse_attn_prefill_blocks", "sparse_attn_decode",
            "sparse_attn_decode_blocks", "sparse_attn_decode_noalloc", "sparse_attn_prefill_paged", "sparse_attn_prefill_chunk", "sparse_attn_prefill_varlen",
            "indexer_project_q",
            "indexer_project_k",
            "acceptance_rate", "acceptance_bin_stats",
            "sparse_attn_profile", "sparse_attn_profile_read", "sparse_attn_peak_mfma", "sparse_attn_peak_stream")
KERNEL_KINDS = ("indexer", "topk", "attention", "merge", "project", "accept")


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class sa_config_t(ctypes.Structure):
    _fields_ = [("n_idx_heads", ctypes.c_int32), ("d_idx", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("v_from_k", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_topk", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("softmax_scale", ctypes.c_float)]


@dataclass(frozen=True)
class Config:
    n_idx_heads: int = 64
    d_idx: int = 128
    n_heads: int = 16
    n_kv_heads: int = 1
    d_qk: int = 576
    d_v: int = 512
    v_from_k: bool = True
    page_size: int = 64
    max_topk: int = 2048
    dtype: str = "bf16"          # element type of q, k, v, q_idx, k_idx: "bf16" or "f32"
    softmax_scale: float = 0.0   # 0 -> 1/sqrt(d_qk)

    def to_c(self) -> sa_config_t:
        return sa_config_t(self.n_idx_heads, self.d_idx, self.n_heads, self.n_kv_heads, self.d_qk,
                           self.d_v, int(self.v_from_k), self.page_size, self.max_topk,
                           SA_BF16 if self.dtype == "bf16" else SA_F32, float(self.softmax_scale))


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libsparse_attn.so (built by ``indexer_selected_sparse_scores_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python indexer_selected_sparse_scores_amd/build.py` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "sparse_attn_create": ([ctypes.POINTER(sa_config_t), ctypes.POINTER(P)], st),
        "sparse_attn_create_host": ([ctypes.POINTER(sa_config_t), i32, ctypes.POINTER(P)], st),
        "sparse_attn_destroy": ([P], None),
        "sparse_attn_last_error": ([P], ctypes.c_char_p),
        "sparse_attn_workspace_size": ([P, ctypes.c_int, i64, i64, ctypes.POINTER(sz)], st),
        "sparse_attn_check": ([P, P, ctypes.POINTER(ctypes.c_uint32)], st),
        "indexer_scores": ([P, P, P, P, i64, P, P], st),
        "topk_select": ([P, P, i64, i64, i64, P, P, i32, P, P], st),
        "topk_select_blocks": ([P, P, i64, i64, i64, P, P, i32, i32, i32, P, P], st),
        "sparse_attn_prefill": ([P, P, P, P, P, P, P, i64, i32, P, P, P, P, sz, P], st),
        "sparse_attn_prefill_blocks": ([P, P, P, P, P, P, P, i64, i32, i32, i32, P, P, P, P, sz, P], st),
        "sparse_attn_decode": ([P, P, P, P, P, P, P, i64, P, i32, P, P, i32, i32, P, P, P, P, sz, P], st),
        "sparse_attn_decode_blocks": ([P, P, P, P, P, P, P, i64, P, i32, P, P, i32, i32, i32, i32, P, P, P, P, sz,
                                       P], st),
        "sparse_attn_decode_noalloc": ([P, P, P, P, P, P, P, i64, P, i32, P, P, i32, i32, P, P, P, P], st),
        "sparse_attn_prefill_paged": ([P, P, P, P, P, P, P, i64, P, i32, i32, P, P, i64, i32, i32, P, P, P, P, sz,
                                       P], st),
        "sparse_attn_prefill_chunk": ([P, P, P, P, P, P, P, i64, P, i32, i64, i64, i32, P, P, P, P, sz, P], st),
        "sparse_attn_prefill_varlen": ([P, P, P, P, P, P, P, i64, P, i32, i32, P, P, i64, i32, i32, P, P, P, P, sz,
                                        P], st),
        "indexer_project_q": ([P, P, i64, P, P, P, P, P, sz, P], st),
        "acceptance_rate": ([P, P, P, i64, i64, i64, P, P, sz, P], st),
        "acceptance_bin_stats": ([P, P, P, i64, i32, i32, ctypes.c_float, P, P, P, P], st),
        "indexer_project_k": ([P, P, i64, P, P, P, i32, i32, i64, P, P, i64, P], st),
        "sparse_attn_peak_mfma": ([P, P, i32, P, P, P], st),
        "sparse_attn_peak_stream": ([P, P, P, i64, P, P], st),
        "sparse_attn_profile": ([P, ctypes.c_int], st),
        "sparse_attn_profile_read": ([P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(t):
    """Device pointer of a tensor (None -> NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(h, status: int):
    if status != SA_OK:
        msg = load_library().sparse_attn_last_error(h)
        raise SparseAttnError(status, msg.decode() if msg else "")


class Handle:
    """Owns an sa_handle_t (created on the current device)."""

    def __init__(self, cfg: Config, host_cus: int | None = None):
        """host_cus: create a host-only planning handle for a device of that many compute units
        (sparse_attn_create_host): calls validate their arguments and launch nothing."""
        lib = load_library()
        self.cfg = cfg
        self._c = cfg.to_c()
        h = ctypes.c_void_p()
        if host_cus is None:
            st = lib.sparse_attn_create(ctypes.byref(self._c), ctypes.byref(h))
        else:
            st = lib.sparse_attn_create_host(ctypes.byref(self._c), int(host_cus), ctypes.byref(h))
        if st != SA_OK:
            raise SparseAttnError(st, lib.sparse_attn_last_error(None).decode())
        self.ptr = h.value

    def close(self):
        if getattr(self, "ptr", None):
            load_library().sparse_attn_destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def sparse_attn_create(cfg: Config) -> Handle:
    return Handle(cfg)


def sparse_attn_destroy(h: Handle) -> None:
    h.close()


def sparse_attn_last_error(h: Handle | None) -> str:
    msg = load_library().sparse_attn_last_error(h.ptr if h else None)
    return msg.decode() if msg else ""


def sparse_attn_workspace_size(h: Handle, op: int, n: int, max_ctx: int = 0) -> int:
    out = ctypes.c_size_t()
    _check(h.ptr, load_library().sparse_attn_workspace_size(h.ptr, op, n, max_ctx, ctypes.byref(out)))
    return out.value


def sparse_attn_check(h: Handle, stream=None) -> int:
    """Synchronise and read the device error word; raises SparseAttnError if set."""
    bits = ctypes.c_uint32()
    _check(h.ptr, load_library().sparse_attn_check(h.ptr, _stream(stream), ctypes.byref(bits)))
    return bits.value


def indexer_scores(h: Handle, q_idx, w, k_idx, scores, stream=None) -> None:
    L = q_idx.shape[0]
    _check(h.ptr, load_library().indexer_scores(h.ptr, _ptr(q_idx), _ptr(w), _ptr(k_idx), L,
                                                _ptr(scores), _stream(stream)))


def topk_select(h: Handle, scores, k: int, idx, valid_len=None, k_per_row=None, cols=None,
                stream=None) -> None:
    rows, ld = scores.shape
    cols = ld if cols is None else cols
    _check(h.ptr, load_library().topk_select(h.ptr, _ptr(scores), rows, cols, ld, _ptr(valid_len),
                                             _ptr(k_per_row), int(k), _ptr(idx), _stream(stream)))


def topk_select_blocks(h: Handle, scores, k: int, block_size: int, n_blocks: int, idx, valid_len=None,
                       k_per_row=None, cols=None, stream=None) -> None:
    """Two-tier selection: n_blocks blocks of block_size tokens kept by their best score, then the
    top-k tokens inside them."""
    rows, ld = scores.shape
    cols = ld if cols is None else cols
    _check(h.ptr, load_library().topk_select_blocks(h.ptr, _ptr(scores), rows, cols, ld, _ptr(valid_len),
                                                    _ptr(k_per_row), int(k), int(block_size), int(n_blocks),
                                                    _ptr(idx), _stream(stream)))


def sparse_attn_prefill(h: Handle, q, k, v, q_idx, w, k_idx, topk: int, out, lse=None,
                        idx_out=None, ws=None, stream=None) -> None:
    L = q.shape[0]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().sparse_attn_prefill(
        h.ptr, _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(w), _ptr(k_idx), L, int(topk), _ptr(out),
        _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_prefill_blocks(h: Handle, q, k, v, q_idx, w, k_idx, topk: int, block_size: int, n_blocks: int,
                               out, lse=None, idx_out=None, ws=None, stream=None) -> None:
    L = q.shape[0]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().sparse_attn_prefill_blocks(
        h.ptr, _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(w), _ptr(k_idx), L, int(topk), int(block_size),
        int(n_blocks), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_decode_blocks(h: Handle, q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table, ctx_len,
                              topk, max_ctx: int, block_size: int, n_blocks: int, out, lse=None, idx_out=None,
                              ws=None, stream=None) -> None:
    B = q.shape[0]
    n_pages = kv_pages.shape[0]
    max_blocks = block_table.shape[1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().sparse_attn_decode_blocks(
        h.ptr, _ptr(q), _ptr(q_idx), _ptr(w), _ptr(kv_pages), _ptr(v_pages), _ptr(kidx_pages), n_pages,
        _ptr(block_table), max_blocks, _ptr(ctx_len), _ptr(topk), B, int(max_ctx), int(block_size),
        int(n_blocks), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_decode(h: Handle, q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table, ctx_len,
                       topk, max_ctx: int, out, lse=None, idx_out=None, ws=None, stream=None) -> None:
    B = q.shape[0]
    n_pages = kv_pages.shape[0]
    max_blocks = block_table.shape[1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().sparse_attn_decode(
        h.ptr, _ptr(q), _ptr(q_idx), _ptr(w), _ptr(kv_pages), _ptr(v_pages), _ptr(kidx_pages), n_pages,
        _ptr(block_table), max_blocks, _ptr(ctx_len), _ptr(topk), B, int(max_ctx), _ptr(out), _ptr(lse),
        _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_decode_noalloc(h: Handle, q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table, ctx_len,
                               topk, max_ctx: int, out, lse=None, idx_out=None, stream=None) -> None:
    """sparse_attn_decode on the library's own device array instead of a workspace (nothing allocated)."""
    B = q.shape[0]
    n_pages = kv_pages.shape[0]
    max_blocks = block_table.shape[1]
    _check(h.ptr, load_library().sparse_attn_decode_noalloc(
        h.ptr, _ptr(q), _ptr(q_idx), _ptr(w), _ptr(kv_pages), _ptr(v_pages), _ptr(kidx_pages), n_pages,
        _ptr(block_table), max_blocks, _ptr(ctx_len), _ptr(topk), B, int(max_ctx), _ptr(out), _ptr(lse),
        _ptr(idx_out), _stream(stream)))


def sparse_attn_prefill_paged(h: Handle, q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table, row_seq, row_pos,
                              max_ctx: int, topk: int, out, lse=None, idx_out=None, ws=None, stream=None) -> None:
    """Query row t is position row_pos[t] of sequence row_seq[t]; it attends over that sequence's
    paged caches (chunked prefill, varlen batches, several new tokens per sequence)."""
    T = q.shape[0]
    n_pages = kv_pages.shape[0]
    n_seqs, max_blocks = block_table.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().sparse_attn_prefill_paged(
        h.ptr, _ptr(q), _ptr(q_idx), _ptr(w), _ptr(kv_pages), _ptr(v_pages), _ptr(kidx_pages), n_pages,
        _ptr(block_table), n_seqs, max_blocks, _ptr(row_seq), _ptr(row_pos), T, int(max_ctx), int(topk), _ptr(out),
        _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_prefill_varlen(h: Handle, q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table, cu_seqlens,
                               ctx_len, max_ctx: int, topk: int, out, lse=None, idx_out=None, ws=None,
                               stream=None) -> None:
    """Sequence b owns query rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1, its newest tokens among its
    ctx_len[b] cached ones (device int32 arrays), over its paged caches."""
    T = q.shape[0]
    n_pages = kv_pages.shape[0]
    n_seqs, max_blocks = block_table.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().sparse_attn_prefill_varlen(
        h.ptr, _ptr(q), _ptr(q_idx), _ptr(w), _ptr(kv_pages), _ptr(v_pages), _ptr(kidx_pages), n_pages,
        _ptr(block_table), n_seqs, max_blocks, _ptr(cu_seqlens), _ptr(ctx_len), T, int(max_ctx), int(topk), _ptr(out),
        _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_prefill_chunk(h: Handle, q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table_row, pos0: int,
                              topk: int, out, lse=None, idx_out=None, ws=None, stream=None) -> None:
    """Rows are the tokens at positions pos0, pos0 + 1, ... of one sequence (block-table row
    block_table_row), over its paged caches."""
    C = q.shape[0]
    n_pages = kv_pages.shape[0]
    max_blocks = block_table_row.shape[-1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().sparse_attn_prefill_chunk(
        h.ptr, _ptr(q), _ptr(q_idx), _ptr(w), _ptr(kv_pages), _ptr(v_pages), _ptr(kidx_pages), n_pages,
        _ptr(block_table_row), max_blocks, int(pos0), C, int(topk), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws),
        ws_bytes, _stream(stream)))


def indexer_project_q(h: Handle, q, W_iq, W_w, q_idx, w, ws=None, stream=None) -> None:
    """q_idx = q W_iq^T (bf16) and w = q W_w^T (fp32) per query row; either pair may be None."""
    L = q.shape[0]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().indexer_project_q(h.ptr, _ptr(q), L, _ptr(W_iq), _ptr(W_w), _ptr(q_idx),
                                                   _ptr(w), _ptr(ws), ws_bytes, _stream(stream)))


def indexer_project_k(h: Handle, k, W_ik, k_idx, block_table=None, n_pages: int = 0, row_seq=None,
                      row_pos=None, pos0: int = 0, stream=None) -> None:
    """k_idx = k W_ik^T per key row, contiguous or into the paged index-key pool (block_table given)."""
    L = k.shape[0]
    n_seqs, max_blocks = (0, 0) if block_table is None else block_table.shape
    _check(h.ptr, load_library().indexer_project_k(h.ptr, _ptr(k), L, _ptr(W_ik), _ptr(k_idx), _ptr(block_table),
                                                   n_seqs, max_blocks, int(n_pages), _ptr(row_seq), _ptr(row_pos),
                                                   int(pos0), _stream(stream)))


def acceptance_rate(h: Handle, logits_p, logits_q, alpha, V: int | None = None, ws=None, stream=None) -> None:
    """alpha[t] = sum_x min(softmax(logits_p[t])(x), softmax(logits_q[t])(x)) over the first V entries.
    ws: a workspace(h, SA_OP_ACCEPT, T, V) tensor for the path that reads each logit once, or None."""
    T, ld = logits_p.shape
    V = ld if V is None else V
    if logits_q.shape != logits_p.shape:
        raise ValueError("logits_p and logits_q must have the same shape")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(h.ptr, load_library().acceptance_rate(h.ptr, _ptr(logits_p), _ptr(logits_q), T, int(V), ld, _ptr(alpha),
                                                 _ptr(ws), ws_bytes, _stream(stream)))


def acceptance_bin_stats(h: Handle, alpha, pos, bin_size: int, n_bins: int, percentile: float, count, mean, pct,
                         stream=None) -> None:
    """Per bin of positions (pos // bin_size): count, mean and the interpolated percentile of alpha."""
    T = alpha.shape[0]
    _check(h.ptr, load_library().acceptance_bin_stats(h.ptr, _ptr(alpha), _ptr(pos), T, int(bin_size), int(n_bins),
                                                      float(percentile), _ptr(count), _ptr(mean), _ptr(pct),
                                                      _stream(stream)))


def sparse_attn_profile(h: Handle, enable: bool) -> None:
    _check(h.ptr, load_library().sparse_attn_profile(h.ptr, int(bool(enable))))


def sparse_attn_profile_read(h: Handle) -> dict:
    """{kernel kind: (summed ms, launches)} since profiling was enabled (synchronises)."""
    ms = (ctypes.c_double * len(KERNEL_KINDS))()
    n = (ctypes.c_int64 * len(KERNEL_KINDS))()
    _check(h.ptr, load_library().sparse_attn_profile_read(h.ptr, ms, n))
    return {k: (ms[i], n[i]) for i, k in enumerate(KERNEL_KINDS)}


def sparse_attn_peak_mfma(h: Handle, operands, iters: int, clocks, sink, stream=None) -> None:
    """Measurement aid: the bf16 MFMA loop on random operands (see the header for the counters)."""
    _check(h.ptr, load_library().sparse_attn_peak_mfma(h.ptr, _ptr(operands), int(iters), _ptr(clocks), _ptr(sink),
                                                       _stream(stream)))


def sparse_attn_peak_stream(h: Handle, src, dst, nbytes: int, sink=None, stream=None) -> None:
    """Measurement aid: a streaming read (dst None) or copy of nbytes."""
    _check(h.ptr, load_library().sparse_attn_peak_stream(h.ptr, _ptr(src), _ptr(dst), int(nbytes), _ptr(sink),
                                                         _stream(stream)))


def workspace(h: Handle, op: int, n: int, max_ctx: int = 0, device=None):
    """A torch uint8 tensor of the size sparse_attn_workspace_size() asks for."""
    import torch
    nbytes = sparse_attn_workspace_size(h, op, n, max_ctx)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device or "cuda")
