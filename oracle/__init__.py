"""CPU oracle for indexer-selected sparse attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It is a slow, plain definition of the method in double precision
(the C part lives in ``oracle.c``, built by ``oracle/build.py``); it shares no code with
the HIP library and never calls it.

What it computes (pages: [P1] "Sparse Attention and RL Optimization: Three Technical
Breakthroughs in LLM Post-Training"; [P3] "Long-Context LLMs Explained: Sparse Attention,
Stable Reinforcement Learning, and Verifiable Synthetic Data"):

* ``indexer_scores`` -- I(t,s) = sum_j w(t,j) ReLU(q(t,j).k(s)), [P1] section 2.2, with the
  causal mask of the [P1] section 2.5 pseudocode (s <= t visible, else -inf).
* ``topk`` -- per query the min(k, visible) keys of largest score, ties to the lower
  index, [P1] section 2.3 / 2.5; padded with -1.
* ``block_topk`` -- the two-tier selection of [P2] "A Guide to Sparse Attention and
  Efficient Reinforcement Learning in LLM Long-Context Inference", section 1.1: a few
  fixed-size blocks kept by their best indexer score, then token-level top-k inside them.
* ``attention_rows`` -- softmax(scale q k_sel^T) v_sel over the selected rows, [P1] section 2.5
  and [P3] section 2.4.
* ``prefill`` -- the three steps above for chosen query rows of one sequence.
* ``decode`` -- one new token per sequence against a paged cache: the pages are first
  laid out contiguously through the block table ([P3] section 2.3: only the selected k
  entries are read, and this composes with paged KV management), then the same steps.
* ``prefill_paged`` -- query rows that each name their sequence and position in paged caches
  (chunked prefill, varlen batches): every row is one decode step of its sequence.
* ``acceptance_rate`` / ``bin_percentiles`` -- the per-token acceptance rate between a dense and a
  sparse next-token distribution and its lower-tail statistic per bin of positions, [P5] "Sparrow:
  Sparse Rollout for Stable and Efficient Long-context RL of Large Language Models", section 3.1.
* ``project`` / ``round_bf16`` / ``paged_slot`` -- the index projections of the [P1] section
  2.5 pseudocode (i_q = W_iq(q), i_k = W_ik(k)) as plain linear maps in double, the rounding
  of their bf16 outputs, and where a projected key lands in the paged index cache.

Parity status: every function is pinned by ``tests/test_oracle_*.py``; none is unpinned.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "oracle.c"))):
        from oracle.build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    lib.orc_indexer_scores.argtypes = [P, P, P, P, i64, i64, ctypes.c_int, ctypes.c_int, P, P]
    lib.orc_indexer_scores.restype = None
    lib.orc_topk.argtypes = [P, i64, P, P, i64, i32, P]
    lib.orc_topk.restype = None
    lib.orc_block_topk.argtypes = [P, i64, P, P, i64, i32, i64, i64, P, P]
    lib.orc_block_topk.restype = None
    lib.orc_attention.argtypes = [P, P, P, P, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_double, P, P]
    lib.orc_attention.restype = None
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_set_num_threads.restype = None
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later OpenMP loops (a timing aid; results do not depend on it)."""
    _load().orc_set_num_threads(int(n))


def default_scale(d_qk: int) -> float:
    """Attention logit scale 1/sqrt(d) of [P1] section 2.5 / [P3] section 2.4, with d the
    key width (d_qk; for the latent layout the value width differs)."""
    return 1.0 / math.sqrt(d_qk)


def decode_budget(n: int, rho: float) -> int:
    """Per-sequence top-k budget that grows with the context, k(n) = min(n, max(256,
    floor(rho n))): the 'k grows slowly with sequence length' knob of [P3] section 2.3,
    in the form the RL-rollout decode sweep workload fixes."""
    return int(min(n, max(256, math.floor(rho * n))))


def indexer_scores(q_idx, w, k_idx, visible, with_abs: bool = False):
    """Scores of n_q query tokens against n_k keys, [P1] section 2.2.

    q_idx [n_q, H_I, d_I], w [n_q, H_I], k_idx [n_k, d_I], visible [n_q] (key s is visible
    to query i iff s < visible[i]).  Returns float64 [n_q, n_k] (-inf where masked), and
    with ``with_abs`` also A = sum_j |w| ReLU(q.k) (the absolute-term sum)."""
    q = _f32(q_idx)
    ww = _f32(w)
    k = _f32(k_idx)
    n_q, H_I, d_I = q.shape
    n_k = k.shape[0]
    assert k.shape == (n_k, d_I) and ww.shape == (n_q, H_I)
    vis = np.ascontiguousarray(np.asarray(visible, dtype=np.int64).reshape(n_q))
    out = np.empty((n_q, n_k), dtype=np.float64)
    absout = np.empty((n_q, n_k), dtype=np.float64) if with_abs else None
    _load().orc_indexer_scores(_ptr(q), _ptr(ww), _ptr(k), _ptr(vis), n_q, n_k, H_I, d_I,
                               _ptr(out), _ptr(absout) if with_abs else None)
    return (out, absout) if with_abs else out


def topk(scores, visible, k_max: int, k_per_row=None) -> np.ndarray:
    """Rank-ordered top-k indices per row, [P1] section 2.3: order the visible keys by
    (score desc, index asc), keep min(k, visible); pad with -1.  int32 [n_q, k_max]."""
    sc = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    if sc.ndim == 1:
        sc = sc[None, :]
    n_q, ld = sc.shape
    vis = np.ascontiguousarray(np.asarray(visible, dtype=np.int64).reshape(n_q))
    assert np.all(vis <= ld)
    kpr = None
    if k_per_row is not None:
        kpr = np.ascontiguousarray(np.asarray(k_per_row, dtype=np.int32).reshape(n_q))
        assert np.all(kpr <= k_max)
    idx = np.empty((n_q, k_max), dtype=np.int32)
    _load().orc_topk(_ptr(sc), ld, _ptr(vis), _ptr(kpr) if kpr is not None else None,
                     n_q, int(k_max), _ptr(idx))
    return idx


def block_topk(scores, visible, k_max: int, block_size: int, n_blocks: int, k_per_row=None,
               with_blocks: bool = False):
    """Two-tier (block -> token) selection, [P2] section 1.1.  Block j is the visible tokens
    s with s // block_size == j; its score is their largest score; the first
    min(n_blocks, visible blocks) blocks by (block score desc, block index asc) are kept;
    the first min(k, candidates) of their tokens by (score desc, index asc) are selected.
    Returns int32 [n_q, k_max] in rank order, -1 padded (and with ``with_blocks`` the kept
    block indices [n_q, n_blocks] in rank order, -1 padded)."""
    assert block_size >= 1 and n_blocks >= 1
    sc = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    if sc.ndim == 1:
        sc = sc[None, :]
    n_q, ld = sc.shape
    vis = np.ascontiguousarray(np.asarray(visible, dtype=np.int64).reshape(n_q))
    assert np.all(vis <= ld)
    kpr = None
    if k_per_row is not None:
        kpr = np.ascontiguousarray(np.asarray(k_per_row, dtype=np.int32).reshape(n_q))
        assert np.all(kpr <= k_max)
    idx = np.empty((n_q, k_max), dtype=np.int32)
    blocks = np.empty((n_q, n_blocks), dtype=np.int32)
    _load().orc_block_topk(_ptr(sc), ld, _ptr(vis), _ptr(kpr) if kpr is not None else None,
                           n_q, int(k_max), int(block_size), int(n_blocks), _ptr(idx), _ptr(blocks))
    return (idx, blocks) if with_blocks else idx


def _select(sc, vis, k_max, k_per_row, blocks):
    """Flat top-k, or the two-tier selection when ``blocks`` = (block_size, n_blocks)."""
    if blocks is None:
        return topk(sc, vis, k_max, k_per_row=k_per_row)
    return block_topk(sc, vis, k_max, blocks[0], blocks[1], k_per_row=k_per_row)


def attention_rows(q, K, V, idx, scale: float, d_v: int | None = None):
    """Softmax attention over the selected rows, [P1] section 2.5 / [P3] section 2.4.

    q [n_q, H, d_qk]; K [n_k, H_kv, d_qk]; V [n_k, H_kv, d_v], or None for the shared latent
    layout where the value is the first ``d_v`` columns of the key row; idx [n_q, k]
    (negative entries are unused slots).  Returns (out [n_q, H, d_v], lse [n_q, H]) in
    float64; a row with no selected key gets out 0 and lse -inf."""
    qq = _f32(q)
    KK = _f32(K)
    n_q, H, d_qk = qq.shape
    n_k, H_kv, d_qk2 = KK.shape
    assert d_qk2 == d_qk and H % H_kv == 0
    if V is None:
        assert d_v is not None and 0 < d_v <= d_qk
        VV = None
    else:
        VV = _f32(V)
        assert VV.shape[:2] == (n_k, H_kv)
        d_v = VV.shape[2]
    ii = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    if ii.ndim == 1:
        ii = ii[None, :]
    assert ii.shape[0] == n_q
    assert ii.size == 0 or ii.max() < n_k
    out = np.empty((n_q, H, d_v), dtype=np.float64)
    lse = np.empty((n_q, H), dtype=np.float64)
    _load().orc_attention(_ptr(qq), _ptr(KK), _ptr(VV) if VV is not None else None, _ptr(ii),
                          ii.shape[1], n_q, n_k, H, H_kv, d_qk, int(d_v), float(scale),
                          _ptr(out), _ptr(lse))
    return out, lse


attention = attention_rows


def prefill(q, K, V, q_idx, w, k_idx, top_k: int, rows=None, scale: float | None = None,
            d_v: int | None = None, with_scores: bool = False, blocks=None):
    """The whole pipeline of [P1] section 2.5 for query rows ``rows`` of one sequence.

    Shapes: q [L,H,d_qk], K [L,H_kv,d_qk], V [L,H_kv,d_v] or None (latent layout, give d_v),
    q_idx [L,H_I,d_I], w [L,H_I], k_idx [L,d_I].  Query row t sees keys s <= t.
    ``blocks`` = (block_size, n_blocks) selects with the two-tier rule of ``block_topk``.
    Returns dict(rows, scores, abs_scores, idx, out, lse); ``scores`` only if asked."""
    q_idx = _f32(q_idx)
    L = q_idx.shape[0]
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    d_qk = np.asarray(q).shape[-1]
    scale = default_scale(d_qk) if scale is None else scale
    vis = rows + 1
    sc, ab = indexer_scores(q_idx[rows], _f32(w)[rows], k_idx, vis, with_abs=True)
    idx = _select(sc, vis, top_k, None, blocks)
    out, lse = attention_rows(_f32(q)[rows], K, V, idx, scale, d_v=d_v)
    res = dict(rows=rows, idx=idx, out=out, lse=lse)
    if with_scores:
        res["scores"] = sc
        res["abs_scores"] = ab
    return res


def depage(pages, block_table_row, n: int) -> np.ndarray:
    """Contiguous view of the first n tokens of one sequence: logical token s lives in
    page block_table_row[s // P], slot s % P, where P is the page size ([P3] section 2.3,
    paged KV management).  pages [n_pages, P, ...]."""
    pg = np.asarray(pages)
    P = pg.shape[1]
    s = np.arange(n, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[s // P]
    assert np.all(blocks >= 0), "block table entry missing for a visible token"
    return pg[blocks, s % P]


def decode(q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table, ctx_len, top_k,
           k_max: int | None = None, seqs=None, scale: float | None = None,
           d_v: int | None = None, with_scores: bool = False, blocks=None):
    """One decode step per sequence against paged caches ([P3] section 2.3).

    q [B,H,d_qk], q_idx [B,H_I,d_I], w [B,H_I]; kv_pages [n_pages,P,H_kv,d_qk];
    v_pages [n_pages,P,H_kv,d_v] or None (latent layout: give d_v); kidx_pages
    [n_pages,P,d_I]; block_table [B, max_blocks]; ctx_len [B] (the new token is the last
    of its n_b visible tokens); top_k int or [B]; ``blocks`` = (block_size, n_blocks) selects
    with the two-tier rule of ``block_topk``.  Returns dict(seqs, idx [nb,k_max],
    out, lse) and, if asked, per-sequence score vectors."""
    q = _f32(q)
    B = q.shape[0]
    d_qk = q.shape[-1]
    scale = default_scale(d_qk) if scale is None else scale
    seqs = np.arange(B) if seqs is None else np.asarray(seqs, dtype=np.int64)
    ks = np.broadcast_to(np.asarray(top_k, dtype=np.int64), (B,))
    k_max = int(ks.max()) if k_max is None else int(k_max)
    idx_all = np.full((len(seqs), k_max), -1, dtype=np.int32)
    H = q.shape[1]
    dv = d_v if v_pages is None else np.asarray(v_pages).shape[-1]
    out_all = np.empty((len(seqs), H, dv), dtype=np.float64)
    lse_all = np.empty((len(seqs), H), dtype=np.float64)
    scores = []
    for r, b in enumerate(seqs):
        n = int(ctx_len[b])
        kI = _f32(depage(kidx_pages, block_table[b], n))
        sc, ab = indexer_scores(_f32(q_idx)[b:b + 1], _f32(w)[b:b + 1], kI, [n], with_abs=True)
        idx = _select(sc, [n], k_max, [int(ks[b])], blocks)
        Kb = _f32(depage(kv_pages, block_table[b], n))
        Vb = None if v_pages is None else _f32(depage(v_pages, block_table[b], n))
        out, lse = attention_rows(q[b:b + 1], Kb, Vb, idx, scale, d_v=d_v)
        idx_all[r] = idx[0]
        out_all[r] = out[0]
        lse_all[r] = lse[0]
        if with_scores:
            scores.append((sc[0], ab[0]))
    res = dict(seqs=seqs, idx=idx_all, out=out_all, lse=lse_all)
    if with_scores:
        res["scores"] = scores
    return res


def prefill_paged(q, q_idx, w, kv_pages, v_pages, kidx_pages, block_table, row_seq, row_pos, top_k: int,
                  rows=None, scale: float | None = None, d_v: int | None = None, with_scores: bool = False):
    """Query rows against paged caches ([P3] section 2.3 with the causal look-back of [P1] section
    2.5): query row t is the token at position p = row_pos[t] of sequence b = row_seq[t] and sees
    the tokens s <= p of b.  Each row is exactly a one-token decode step of sequence b with context
    p + 1, so this is ``decode`` over the rows, each given its sequence's block-table row.
    Returns the dict of ``decode`` for the chosen rows (all by default)."""
    rs = np.asarray(row_seq, dtype=np.int64)
    rp = np.asarray(row_pos, dtype=np.int64)
    rows = np.arange(len(rs)) if rows is None else np.asarray(rows, dtype=np.int64)
    table = np.asarray(block_table)[rs[rows]]
    res = decode(_f32(q)[rows], _f32(q_idx)[rows], _f32(w)[rows], kv_pages, v_pages, kidx_pages, table,
                 rp[rows] + 1, top_k, k_max=top_k, scale=scale, d_v=d_v, with_scores=with_scores)
    res["rows"] = rows
    return res


# ---------------------------------------------------------------------------------------
# Acceptance rate between dense and sparse next-token distributions
# ---------------------------------------------------------------------------------------
def softmax(logits) -> np.ndarray:
    """Row-wise softmax in float64 (max subtracted first)."""
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def acceptance_rate(logits_p, logits_q) -> np.ndarray:
    """Per-token acceptance rate, [P5] section 3.1: with p and q the softmax distributions of the
    two logit rows over the vocabulary, alpha = E_{x~q}[min(p(x)/q(x), 1)] = sum_x min(p(x), q(x))
    (the page prints the right-hand side as an expectation over the vocabulary; the sum is what the
    left-hand side equals).  logits [T, V] -> alpha [T] float64."""
    return np.minimum(softmax(logits_p), softmax(logits_q)).sum(axis=-1)


def bin_percentiles(alpha, pos, bin_size: int, n_bins: int, percentile: float):
    """Lower-tail statistic per bin of positions, [P5] section 3.1 (the 5-percentile of the
    per-token acceptance rate in bins of 2K positions): token t falls in bin pos[t] // bin_size
    (tokens outside [0, n_bins) are ignored).  Per bin: the count, the mean and the percentile of
    its values, the percentile taken between order statistics as
    h = (n - 1) percentile / 100, x[floor h] + (h - floor h) (x[floor h + 1] - x[floor h]) on the
    ascending values x (NaN for an empty bin).  Returns (count int64, mean, pct) float64 arrays."""
    a = np.asarray(alpha, dtype=np.float64)
    b = np.asarray(pos, dtype=np.int64) // int(bin_size)
    count = np.zeros(n_bins, dtype=np.int64)
    mean = np.full(n_bins, np.nan)
    pct = np.full(n_bins, np.nan)
    for j in range(n_bins):
        x = np.sort(a[b == j])
        n = len(x)
        count[j] = n
        if n == 0:
            continue
        mean[j] = x.sum() / n
        h = (n - 1) * percentile / 100.0
        lo = int(math.floor(h))
        hi = min(lo + 1, n - 1)
        pct[j] = x[lo] + (h - lo) * (x[hi] - x[lo])
    return count, mean, pct


# ---------------------------------------------------------------------------------------
# Index-space projections
# ---------------------------------------------------------------------------------------
def project(x, W) -> np.ndarray:
    """Row-wise linear map y[t] = W x[t] in double: the index projections of the [P1] section 2.5
    pseudocode (i_q = W_iq(q), i_k = W_ik(k)); the head weights w(t, j) of the [P1] section 2.2
    score are read as one more such map of the query row.  x [L, in], W [out, in] -> [L, out].
    A library matmul serves as the step."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def project_abs(x, W) -> np.ndarray:
    """sum_c |W[o, c] x[t, c]|: the size of the terms behind each projected value (tolerances)."""
    return np.abs(np.asarray(x, dtype=np.float64)) @ np.abs(np.asarray(W, dtype=np.float64)).T


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits), ties to even, of finite doubles in bf16's normal
    range: x = m 2^e with 0.5 <= |m| < 1, and m is rounded to a multiple of 2^-8."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def paged_slot(block_table, seq: int, pos: int, page_size: int, n_pages: int):
    """(page, slot) of position pos of sequence seq in a paged cache ([P3] section 2.3, paged KV
    management): page block_table[seq][pos // page_size], slot pos % page_size; None when the
    position or its page entry is out of range."""
    bt = np.asarray(block_table)
    if pos < 0 or seq < 0 or seq >= bt.shape[0] or pos // page_size >= bt.shape[1]:
        return None
    page = int(bt[seq, pos // page_size])
    if page < 0 or page >= n_pages:
        return None
    return page, pos % page_size
