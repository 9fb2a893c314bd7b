"""GPU parity of query rows against paged caches (sparse_attn_prefill_paged): chunked prefill,
varlen batches and several new tokens per sequence, against the CPU oracle.

Pages: "Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and
Verifiable Synthetic Data", section 2.3 (selection over a paged cache), with the causal look-back
of "Sparse Attention and RL Optimization: Three Technical Breakthroughs in LLM Post-Training",
section 2.5.  Tolerances are those of tests/parity.py."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import indexer_selected_sparse_scores_amd as sa
import oracle
from indexer_selected_sparse_scores_amd import inputs
from tests.parity import check_attention, check_topk_row, compact_pages, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _run(h, d, topk, max_ctx=None, check=True):
    T = d["q"].shape[0]
    s = h.cfg
    max_ctx = int(d["rp_np"].max()) + 1 if max_ctx is None else max_ctx
    out = torch.empty((T, s.n_heads, s.d_v), device=DEV, dtype=torch.float32)
    lse = torch.empty((T, s.n_heads), device=DEV, dtype=torch.float32)
    idx = torch.empty((T, topk), device=DEV, dtype=torch.int32)
    ws = sa.workspace(h, sa.SA_OP_PREFILL_PAGED, T, max_ctx)
    sa.sparse_attn_prefill_paged(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], d["v_pages"], d["kidx_pages"],
                                 d["block_table"], d["row_seq"], d["row_pos"], max_ctx, topk, out, lse, idx, ws)
    if check:
        assert sa.sparse_attn_check(h) == 0
    return out, lse, idx


def _check(d, out, lse, idx, rows, topk, d_v, what, latent=True):
    """Sampled rows against the oracle: selection with the near-tie rule, attention on the GPU's
    own selection.  Pages leave the device once per sequence."""
    rows = np.asarray(sorted(set(int(r) for r in rows)))
    rs, rp = d["rs_np"], d["rp_np"]
    table = to_np(d["block_table"])
    gi = to_np(idx)
    q, qi, w = to_np(d["q"]), to_np(d["q_idx"]), to_np(d["w"])
    diffs = 0
    ref_out = np.empty((len(rows), q.shape[1], d_v))
    ref_lse = np.empty((len(rows), q.shape[1]))
    for b in np.unique(rs[rows]):
        mine = [i for i, t in enumerate(rows) if rs[t] == b]
        n_max = int(rp[rows[mine]].max()) + 1
        kv_pool, tab = compact_pages(d["kv_pages"], table[b:b + 1], np.array([n_max]))
        ki_pool, _ = compact_pages(d["kidx_pages"], table[b:b + 1], np.array([n_max]))
        v_pool = None if latent else compact_pages(d["v_pages"], table[b:b + 1], np.array([n_max]))[0]
        for i in mine:
            t = rows[i]
            n = int(rp[t]) + 1
            kI = oracle.depage(ki_pool, tab[0], n)
            sc = oracle.indexer_scores(qi[t:t + 1], w[t:t + 1], kI, [n])[0]
            diffs += check_topk_row(gi[t], sc, min(topk, n), n, what=f"{what} row {t} (seq {b}, pos {n - 1})")
            Kb = oracle.depage(kv_pool, tab[0], n)
            Vb = None if latent else oracle.depage(v_pool, tab[0], n)
            o, l = oracle.attention_rows(q[t:t + 1], Kb, Vb, gi[t:t + 1], oracle.default_scale(q.shape[-1]), d_v=d_v)
            ref_out[i], ref_lse[i] = o[0], l[0]
    err = check_attention(to_np(out)[rows], to_np(lse)[rows], ref_out, ref_lse, what=what)
    say(f"{what}: rows={len(rows)} near-tie set diffs={diffs} max|dO|={err:.2e}")


def test_chunked_prefill_of_one_sequence():
    """The last 1000 tokens of a 3000-token paged sequence as one chunk, rows shuffled (one
    attention workgroup per row)."""
    wl = inputs.WORKLOADS["decode_b64"]
    n = 3000
    pos = np.random.default_rng(1).permutation(np.arange(2000, n))
    say(f"prefill_paged chunk: positions 2000..2999 of a {n}-token sequence, topk=256")
    d = inputs.paged_rows_inputs(inputs.small(wl, topk=256), [n], np.zeros(len(pos), np.int64), pos, DEV, seed=21)
    with sa.Handle(inputs.library_config(wl, max_topk=256)) as h:
        out, lse, idx = _run(h, d, 256)
    rows = np.concatenate([np.arange(8), np.argsort(pos)[[0, 1, -2, -1]],
                           np.random.default_rng(2).integers(0, len(pos), 20)])
    _check(d, out, lse, idx, rows, 256, 512, "prefill_paged chunk")


def test_varlen_batch_every_position():
    """Four sequences (700, 64, 1500 and 1 tokens), every position of each as a query row, rows
    interleaved; k = 512 exceeds the short sequences, which fall back to dense attention."""
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [700, 64, 1500, 1]
    rs = np.concatenate([np.full(n, b) for b, n in enumerate(ctx)])
    rp = np.concatenate([np.arange(n) for n in ctx])
    order = np.random.default_rng(3).permutation(len(rs))
    rs, rp = rs[order], rp[order]
    say(f"prefill_paged varlen ctx={ctx} T={len(rs)} topk=512")
    d = inputs.paged_rows_inputs(inputs.small(wl, topk=512), ctx, rs, rp, DEV, seed=22)
    with sa.Handle(inputs.library_config(wl, max_topk=512)) as h:
        out, lse, idx = _run(h, d, 512)
    where = {(int(b), int(p)): t for t, (b, p) in enumerate(zip(rs, rp))}
    picks = [(0, 0), (0, 511), (0, 512), (0, 699), (1, 0), (1, 63), (2, 0), (2, 513), (2, 1024), (2, 1499), (3, 0)]
    rows = [where[k] for k in picks] + list(np.random.default_rng(4).integers(0, len(rs), 16))
    _check(d, out, lse, idx, rows, 512, 512, "prefill_paged varlen")


def test_one_row_per_sequence_equals_decode():
    """Rows at the last position of each sequence are decode steps: bit-identical to
    sparse_attn_decode on the same rows (few rows: the split attention path)."""
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [5000, 129, 20000, 64, 777, 4097, 3, 16384]
    B = len(ctx)
    say(f"prefill_paged one row per sequence vs sparse_attn_decode, ctx={ctx}")
    d = inputs.paged_rows_inputs(inputs.small(wl, topk=2048), ctx, np.arange(B), np.array(ctx) - 1, DEV, seed=23)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _run(h, d, 2048)
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        idx2 = torch.empty_like(idx)
        ws = sa.workspace(h, sa.SA_OP_DECODE, B, d["max_ctx"])
        sa.sparse_attn_decode(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], None, d["kidx_pages"], d["block_table"],
                              d["ctx_len"], d["topk"], d["max_ctx"], out2, lse2, idx2, ws)
        assert sa.sparse_attn_check(h) == 0
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)
    _check(d, out, lse, idx, np.arange(B), 2048, 512, "prefill_paged = decode")


def test_generic_kernels_fp32():
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], shapes=inputs.TINY, topk=16)
    ctx = [100, 333]
    rs = np.concatenate([np.full(n, b) for b, n in enumerate(ctx)])
    rp = np.concatenate([np.arange(n) for n in ctx])
    say(f"prefill_paged tiny (fp32, generic kernels) ctx={ctx} T={len(rs)} topk=16")
    d = inputs.paged_rows_inputs(wl, ctx, rs, rp, DEV, seed=24)
    with sa.Handle(inputs.library_config(wl, max_topk=16)) as h:
        out, lse, idx = _run(h, d, 16)
    _check(d, out, lse, idx, np.arange(len(rs)), 16, 64, "prefill_paged tiny", latent=False)


def test_bad_rows_are_flagged_and_skipped():
    """A row naming a sequence or position out of range sets SA_DEVERR_ROW; the other rows are
    unaffected."""
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [300, 200]
    rs = np.array([0, 1, 0, 1, 0])
    rp = np.array([10, 199, 299, 5, 150])
    say("prefill_paged with a bad sequence id and a bad position")
    d = inputs.paged_rows_inputs(inputs.small(wl, topk=64), ctx, rs, rp, DEV, seed=25)
    bad_seq = d["row_seq"].clone()
    bad_seq[1] = 7          # only 2 sequences
    bad_pos = d["row_pos"].clone()
    bad_pos[3] = 400        # beyond max_ctx = 300
    d2 = dict(d, row_seq=bad_seq, row_pos=bad_pos)
    with sa.Handle(inputs.library_config(wl, max_topk=64)) as h:
        out, lse, idx = _run(h, d2, 64, max_ctx=300, check=False)
        bits = ctypes.c_uint32()
        st = sa.load_library().sparse_attn_check(h.ptr, torch.cuda.current_stream().cuda_stream, ctypes.byref(bits))
        assert st == sa.SA_ERR_DEVICE_CHECK
        assert bits.value & sa.SA_DEVERR_ROW
        assert sa.sparse_attn_check(h) == 0  # cleared
    _check(d, out, lse, idx, [0, 2, 4], 64, 512, "prefill_paged good rows beside bad ones")


def test_chunk_at_128k():
    """The chunk the benchmark times: the last 2048 positions of a 131072-token paged sequence."""
    wl = inputs.WORKLOADS["decode_b64"]
    n, T = 131072, 2048
    say(f"prefill_paged chunk of {T} at the end of a {n}-token sequence, topk=2048 (5 rows checked)")
    d = inputs.paged_rows_inputs(wl, [n], np.zeros(T, np.int64), np.arange(n - T, n), DEV, seed=26)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _run(h, d, 2048)
    _check(d, out, lse, idx, [0, 1, 1000, T - 2, T - 1], 2048, 512, "prefill_paged 128k chunk")
    del d, out, lse, idx
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------
# sparse_attn_prefill_chunk: one sequence, rows at positions pos0 .. pos0 + C - 1
# ---------------------------------------------------------------------------------------
def _run_chunk(h, d, pos0, C, topk, table_row=0, rows=None, check=True):
    s = h.cfg
    sl = slice(None) if rows is None else rows
    q, qi, w = d["q"][sl], d["q_idx"][sl], d["w"][sl]
    out = torch.empty((C, s.n_heads, s.d_v), device=DEV, dtype=torch.float32)
    lse = torch.empty((C, s.n_heads), device=DEV, dtype=torch.float32)
    idx = torch.empty((C, topk), device=DEV, dtype=torch.int32)
    ws = sa.workspace(h, sa.SA_OP_PREFILL_CHUNK, C, pos0 + C)
    sa.sparse_attn_prefill_chunk(h, q.contiguous(), qi.contiguous(), w.contiguous(), d["kv_pages"], d["v_pages"],
                                 d["kidx_pages"], d["block_table"][table_row].contiguous(), pos0, topk, out, lse, idx,
                                 ws)
    if check:
        assert sa.sparse_attn_check(h) == 0
    return out, lse, idx


def test_chunk_of_one_sequence_matches_the_oracle():
    """Positions 2000..2999 of a 3000-token paged sequence through the fused row tiles."""
    wl = inputs.WORKLOADS["decode_b64"]
    n, pos0 = 3000, 2000
    say(f"prefill_chunk: positions {pos0}..{n - 1} of a {n}-token sequence, topk=256")
    pos = np.arange(pos0, n)
    d = inputs.paged_rows_inputs(inputs.small(wl, topk=256), [n], np.zeros(len(pos), np.int64), pos, DEV, seed=31)
    with sa.Handle(inputs.library_config(wl, max_topk=256)) as h:
        out, lse, idx = _run_chunk(h, d, pos0, len(pos), 256)
    rows = np.concatenate([np.arange(6), [len(pos) - 2, len(pos) - 1], np.random.default_rng(5).integers(0, len(pos), 20)])
    _check(d, out, lse, idx, rows, 256, 512, "prefill_chunk")


def test_chunks_equal_the_contiguous_prefill_bit_for_bit():
    """Two chunks (0..1499, 1500..2999) over shuffled pages give exactly what sparse_attn_prefill gives on
    the same sequence laid out contiguously: the same fused kernel, the same keys in the same order."""
    wl = inputs.WORKLOADS["prefill_8k"]
    L, split = 3000, 1500
    say(f"prefill_chunk x2 vs sparse_attn_prefill, L={L}, topk=512")
    P = inputs.prefill_inputs(wl, DEV, L=L)
    page = 64
    n_pages = (L + page - 1) // page
    perm = torch.from_numpy(np.random.default_rng(6).permutation(n_pages).astype(np.int64)).to(DEV)
    pad = n_pages * page - L
    k_pad = torch.cat([P["k"].reshape(L, -1), torch.zeros((pad, P["k"].shape[-1] * P["k"].shape[1]), dtype=P["k"].dtype,
                                                            device=DEV)])
    ki_pad = torch.cat([P["k_idx"], torch.zeros((pad, P["k_idx"].shape[1]), dtype=P["k_idx"].dtype, device=DEV)])
    kv_pages = torch.empty((n_pages, page, 1, k_pad.shape[1]), dtype=k_pad.dtype, device=DEV)
    kidx_pages = torch.empty((n_pages, page, ki_pad.shape[1]), dtype=ki_pad.dtype, device=DEV)
    kv_pages[perm] = k_pad.reshape(n_pages, page, 1, -1)
    kidx_pages[perm] = ki_pad.reshape(n_pages, page, -1)
    table = perm.to(torch.int32).reshape(1, -1)
    d = {"q": P["q"], "q_idx": P["q_idx"], "w": P["w"], "kv_pages": kv_pages, "v_pages": None,
         "kidx_pages": kidx_pages, "block_table": table}
    with sa.Handle(inputs.library_config(wl, max_topk=512)) as h:
        o1, l1, i1 = _run_chunk(h, d, 0, split, 512, rows=slice(0, split))
        o2, l2, i2 = _run_chunk(h, d, split, L - split, 512, rows=slice(split, L))
        out = torch.empty((L, 16, 512), device=DEV)
        lse = torch.empty((L, 16), device=DEV)
        idx = torch.empty((L, 512), device=DEV, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_PREFILL, L)
        sa.sparse_attn_prefill(h, P["q"], P["k"], None, P["q_idx"], P["w"], P["k_idx"], 512, out, lse, idx, ws)
        assert sa.sparse_attn_check(h) == 0
    assert torch.equal(torch.cat([i1, i2]), idx)
    assert torch.equal(torch.cat([o1, o2]), out)
    assert torch.equal(torch.cat([l1, l2]), lse)


def test_chunk_generic_kernels_fp32():
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], shapes=inputs.TINY, topk=16)
    n, pos0 = 333, 200
    say(f"prefill_chunk tiny (fp32, generic kernels): positions {pos0}..{n - 1}, topk=16")
    pos = np.arange(pos0, n)
    d = inputs.paged_rows_inputs(wl, [n], np.zeros(len(pos), np.int64), pos, DEV, seed=32)
    with sa.Handle(inputs.library_config(wl, max_topk=16)) as h:
        out, lse, idx = _run_chunk(h, d, pos0, len(pos), 16)
    _check(d, out, lse, idx, np.arange(len(pos)), 16, 64, "prefill_chunk tiny", latent=False)


def test_chunk_with_a_bad_page_entry():
    """A bad block-table entry among the visible pages is flagged; its tokens get no weight and every
    other token is unaffected (rows before that page are exact)."""
    wl = inputs.WORKLOADS["decode_b64"]
    n, pos0 = 1000, 600
    say("prefill_chunk with a corrupted block-table entry (page 3)")
    pos = np.arange(pos0, n)
    d = inputs.paged_rows_inputs(inputs.small(wl, topk=64), [n], np.zeros(len(pos), np.int64), pos, DEV, seed=33)
    bt = d["block_table"].clone()
    bt[0, 3] = 10 ** 6
    d2 = dict(d, block_table=bt)
    with sa.Handle(inputs.library_config(wl, max_topk=64)) as h:
        out, lse, idx = _run_chunk(h, d2, pos0, len(pos), 64, check=False)
        bits = ctypes.c_uint32()
        st = sa.load_library().sparse_attn_check(h.ptr, torch.cuda.current_stream().cuda_stream, ctypes.byref(bits))
        assert st == sa.SA_ERR_DEVICE_CHECK and bits.value & sa.SA_DEVERR_BLOCK_TABLE
    assert torch.isfinite(out).all()
    gi = to_np(idx)
    # a selected token of the bad page (192..255) can only be there as a -inf score, i.e. never while
    # enough finite ones exist
    assert not np.any((gi >= 192) & (gi < 256))


def test_prefill_chunk_at_128k():
    """The chunk the benchmark times through the fused row tiles: the last 4096 positions of a 131072-token
    paged sequence."""
    wl = inputs.WORKLOADS["decode_b64"]
    n, C = 131072, 4096
    say(f"prefill_chunk of {C} at the end of a {n}-token sequence, topk=2048 (5 rows checked)")
    d = inputs.paged_rows_inputs(wl, [n], np.zeros(C, np.int64), np.arange(n - C, n), DEV, seed=34)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _run_chunk(h, d, n - C, C, 2048)
    _check(d, out, lse, idx, [0, 1, 2000, C - 2, C - 1], 2048, 512, "prefill_chunk 128k")
    del d, out, lse, idx
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------
# sparse_attn_prefill_varlen: contiguous rows per sequence, layout on the device only
# ---------------------------------------------------------------------------------------
def _varlen(ctx, n_new, topk, seed):
    """Sequence b's n_new[b] newest tokens as its contiguous rows; cu_seqlens and ctx_len on the device."""
    rs = np.concatenate([np.full(k, b) for b, k in enumerate(n_new)])
    rp = np.concatenate([np.arange(c - k, c) for c, k in zip(ctx, n_new)])
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], topk=topk)
    d = inputs.paged_rows_inputs(wl, ctx, rs, rp, DEV, seed=seed)
    d["cu"] = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).to(DEV)
    d["ctx_len"] = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).to(DEV)
    return wl, d


def _run_varlen(h, d, topk, max_ctx, check=True):
    T = d["q"].shape[0]
    s = h.cfg
    out = torch.empty((T, s.n_heads, s.d_v), device=DEV, dtype=torch.float32)
    lse = torch.empty((T, s.n_heads), device=DEV, dtype=torch.float32)
    idx = torch.empty((T, topk), device=DEV, dtype=torch.int32)
    ws = sa.workspace(h, sa.SA_OP_PREFILL_VARLEN, T, max_ctx)
    sa.sparse_attn_prefill_varlen(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], d["v_pages"], d["kidx_pages"],
                                  d["block_table"], d["cu"], d["ctx_len"], max_ctx, topk, out, lse, idx, ws)
    if check:
        assert sa.sparse_attn_check(h) == 0
    return out, lse, idx


def test_varlen_row_tiles_match_the_oracle():
    """Six sequences with ragged new-row counts (a full 700-token prefill, tails of 1, 9 and 13 rows, a
    1-token sequence) on the fused row tiles, k = 512."""
    ctx, n_new = [3000, 700, 64, 1500, 2049, 1], [1000, 700, 13, 9, 1, 1]
    say(f"prefill_varlen ctx={ctx} new={n_new} topk=512")
    wl, d = _varlen(ctx, n_new, 512, seed=31)
    with sa.Handle(inputs.library_config(wl, max_topk=512)) as h:
        out, lse, idx = _run_varlen(h, d, 512, max(ctx))
    cu = np.concatenate([[0], np.cumsum(n_new)])
    rows = [0, 1, 7, 8, 511, 999, 1000, 1511, 1512, 1699, 1700, 1712, 1713, 1721, 1722, 1723]
    rows += list(np.random.default_rng(5).integers(0, int(cu[-1]), 16))
    _check(d, out, lse, idx, rows, 512, 512, "prefill_varlen")


def test_varlen_one_sequence_equals_the_chunk_bit_for_bit():
    """One sequence's last 1000 tokens: the varlen call and the chunk call run the same row tiles."""
    n, C = 5000, 1000
    say(f"prefill_varlen vs prefill_chunk: positions {n - C}..{n - 1} of {n}, topk=2048")
    wl, d = _varlen([n], [C], 2048, seed=32)
    s = inputs.library_config(wl, max_topk=2048)
    with sa.Handle(s) as h:
        out, lse, idx = _run_varlen(h, d, 2048, n)
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        idx2 = torch.empty_like(idx)
        ws = sa.workspace(h, sa.SA_OP_PREFILL_CHUNK, C, n)
        sa.sparse_attn_prefill_chunk(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], d["v_pages"], d["kidx_pages"],
                                     d["block_table"][0], n - C, 2048, out2, lse2, idx2, ws)
        assert sa.sparse_attn_check(h) == 0
    assert torch.equal(idx, idx2), "selections differ"
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "outputs differ"


def test_varlen_bad_layout_is_flagged():
    """cu_seqlens that decrease: the device flags SA_DEVERR_ROW, and the rows of no valid sequence
    get empty selections."""
    ctx, n_new = [300, 200], [100, 50]
    say("prefill_varlen with a decreasing cu_seqlens")
    wl, d = _varlen(ctx, n_new, 64, seed=33)
    d["cu"] = torch.tensor([0, 120, 100], dtype=torch.int32, device=DEV)  # sequence 1 has -20 rows
    with sa.Handle(inputs.library_config(wl, max_topk=64)) as h:
        out, lse, idx = _run_varlen(h, d, 64, max(ctx), check=False)
        bits = ctypes.c_uint32()
        st = sa.load_library().sparse_attn_check(h.ptr, torch.cuda.current_stream().cuda_stream, ctypes.byref(bits))
        assert st == sa.SA_ERR_DEVICE_CHECK
        assert bits.value & sa.SA_DEVERR_ROW, bits.value
        assert sa.sparse_attn_check(h) == 0  # cleared
    gi = to_np(idx)
    assert np.all(gi[120:] == -1), "rows outside every valid sequence must select nothing"


def test_varlen_generic_kernels_fp32():
    """An fp32 handle takes the varlen call's other path: the device row layout, then the rows as
    sparse_attn_prefill_paged rows (generic kernels), against the oracle on every row."""
    ctx, n_new = [100, 333, 7], [40, 333, 7]
    rs = np.concatenate([np.full(k, b) for b, k in enumerate(n_new)])
    rp = np.concatenate([np.arange(c - k, c) for c, k in zip(ctx, n_new)])
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], shapes=inputs.TINY, topk=16)
    say(f"prefill_varlen tiny (fp32, generic path) ctx={ctx} new={n_new} topk=16")
    d = inputs.paged_rows_inputs(wl, ctx, rs, rp, DEV, seed=35)
    d["cu"] = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).to(DEV)
    d["ctx_len"] = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).to(DEV)
    with sa.Handle(inputs.library_config(wl, max_topk=16)) as h:
        out, lse, idx = _run_varlen(h, d, 16, max(ctx))
    _check(d, out, lse, idx, np.arange(len(rs)), 16, 64, "prefill_varlen tiny", latent=False)


def test_varlen_few_rows_split_attention():
    """Fewer rows than compute units: the fused row tiles, then the split decode attention over the varlen
    rows.  Eight sequences with 0 to 4 new rows each (one sequence contributes none)."""
    ctx, n_new = [900, 5000, 64, 2049, 3000, 1, 700, 4100], [3, 4, 0, 1, 2, 1, 4, 2]
    say(f"prefill_varlen few rows ctx={ctx} new={n_new} topk=2048")
    wl, d = _varlen(ctx, n_new, 2048, seed=36)
    with sa.Handle(inputs.library_config(wl, max_topk=2048)) as h:
        out, lse, idx = _run_varlen(h, d, 2048, max(ctx))
    _check(d, out, lse, idx, np.arange(sum(n_new)), 2048, 512, "prefill_varlen few rows")


def test_varlen_at_128k_sampled():
    """The varlen batch the benchmark times: 8 sequences of 131072 cached tokens, the last 512 of each as
    new rows; 4 rows of each sequence checked."""
    n, per, n_seq = 131072, 512, 8
    say(f"prefill_varlen {n_seq} x {per} new rows at the end of {n}-token contexts (32 rows checked)")
    wl, d = _varlen([n] * n_seq, [per] * n_seq, 2048, seed=37)
    with sa.Handle(inputs.library_config(wl, max_topk=2048)) as h:
        out, lse, idx = _run_varlen(h, d, 2048, n)
    rows = [b * per + r for b in range(n_seq) for r in (0, 1, per // 2 + b, per - 1)]
    _check(d, out, lse, idx, rows, 2048, 512, "prefill_varlen 128k")
    del d, out, lse, idx
    torch.cuda.empty_cache()


def test_row_tiles_and_per_row_path_agree_bit_for_bit():
    """Up to 16384 rows run as fused row tiles (sorted by sequence and position on the device); one more
    row sends the same call down the per-row path (decode indexer and top-k per row).  Both compute the
    same scores in the same order, so on the shared rows every selection and output is bit-identical; a
    sample is also checked against the oracle.  Rows come from 40 sequences, interleaved and shuffled."""
    wl = inputs.WORKLOADS["decode_b64"]
    n_seq, T = 40, 16385
    rng = np.random.default_rng(38)
    ctx = rng.integers(200, 3000, n_seq)
    rs = rng.integers(0, n_seq, T)
    rp = np.array([rng.integers(0, ctx[b]) for b in rs])
    say(f"prefill_paged: {T - 1} rows as row tiles vs {T} rows per row, {n_seq} sequences, topk=128")
    d = inputs.paged_rows_inputs(inputs.small(wl, topk=128), ctx, rs, rp, DEV, seed=38)
    with sa.Handle(inputs.library_config(wl, max_topk=128)) as h:
        out, lse, idx = _run(h, d, 128)
        part = {k: (v[:T - 1] if isinstance(v, torch.Tensor) and v.shape[:1] == (T,) else v) for k, v in d.items()}
        part["rp_np"] = rp[:T - 1]
        out2, lse2, idx2 = _run(h, part, 128, max_ctx=int(rp.max()) + 1)
    assert torch.equal(idx[:T - 1], idx2), "selections differ between the two paths"
    assert torch.equal(out[:T - 1], out2) and torch.equal(lse[:T - 1], lse2), "outputs differ between the two paths"
    _check(d, out, lse, idx, rng.integers(0, T, 24), 128, 512, "prefill_paged row tiles / per row")
