"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Each test prints the case it runs before touching the GPU.  Tolerances are in
tests/parity.py.  Pages: "Sparse Attention and RL Optimization: Three Technical
Breakthroughs in LLM Post-Training" (sections 2.2, 2.3, 2.5) and "Long-Context LLMs
Explained: Sparse Attention, Stable Reinforcement Learning, and Verifiable Synthetic Data"
(sections 2.3, 2.4)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import indexer_selected_sparse_scores_amd as sa
import oracle
from indexer_selected_sparse_scores_amd import inputs
from tests.parity import (check_attention, check_scores, check_topk_row, compact_pages, to_np)

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


def _prefill(h, d, topk, want_lse=True):
    L = d["q"].shape[0]
    s = h.cfg
    out = torch.empty((L, s.n_heads, s.d_v), device=DEV, dtype=torch.float32)
    lse = torch.empty((L, s.n_heads), device=DEV, dtype=torch.float32) if want_lse else None
    idx = torch.empty((L, topk), device=DEV, dtype=torch.int32)
    ws = sa.workspace(h, sa.SA_OP_PREFILL, L)
    sa.sparse_attn_prefill(h, d["q"], d["k"], d["v"], d["q_idx"], d["w"], d["k_idx"], topk, out, lse,
                           idx, ws)
    assert sa.sparse_attn_check(h) == 0
    return out, lse, idx


def _check_prefill_rows(d, out, lse, idx, topk, rows, latent, d_v, what):
    rows = np.asarray(rows, dtype=np.int64)
    rt = torch.as_tensor(rows, device=d["q"].device)
    sub = lambda t: to_np(t[rt])  # only the sampled rows leave the device
    sc = oracle.indexer_scores(sub(d["q_idx"]), sub(d["w"]), to_np(d["k_idx"]), rows + 1)
    gi = sub(idx)
    diffs = 0
    for i, t in enumerate(rows):
        m = min(topk, t + 1)
        diffs += check_topk_row(gi[i], sc[i], m, t + 1, what=f"{what} row {t}")
    ref_out, ref_lse = oracle.attention_rows(sub(d["q"]), to_np(d["k"]),
                                             None if latent else to_np(d["v"]), gi,
                                             oracle.default_scale(d["q"].shape[-1]), d_v=d_v)
    err = check_attention(sub(out), None if lse is None else sub(lse), ref_out, ref_lse, what=what)
    say(f"{what}: rows={len(rows)} near-tie set diffs={diffs} max|dO|={err:.2e}")
    return diffs


# ---------------------------------------------------------------------------------------
# indexer_scores
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("wl_name,L", [("tiny_prefill", 256), ("prefill_8k", 300), ("prefill_8k", 1029)])
def test_indexer_scores_full(wl_name, L):
    wl = inputs.WORKLOADS[wl_name]
    say(f"indexer_scores {wl_name} L={L}")
    d = inputs.prefill_inputs(wl, DEV, L=L)
    with sa.Handle(inputs.library_config(wl)) as h:
        scores = torch.empty((L, L), device=DEV, dtype=torch.float32)
        sa.indexer_scores(h, d["q_idx"], d["w"], d["k_idx"], scores)
        assert sa.sparse_attn_check(h) == 0
        ref, ref_abs = oracle.indexer_scores(to_np(d["q_idx"]), to_np(d["w"]), to_np(d["k_idx"]),
                                             np.arange(1, L + 1), with_abs=True)
        check_scores(to_np(scores), ref, ref_abs, what=f"{wl_name} L={L}")


def test_indexer_scores_8k_sampled_rows():
    wl = inputs.WORKLOADS["prefill_8k"]
    L = wl.L
    say(f"indexer_scores prefill_8k L={L} (sampled rows)")
    d = inputs.prefill_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl)) as h:
        scores = torch.empty((L, L), device=DEV, dtype=torch.float32)
        sa.indexer_scores(h, d["q_idx"], d["w"], d["k_idx"], scores)
        assert sa.sparse_attn_check(h) == 0
        rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, L - 2, L - 1],
                                         np.random.default_rng(5).integers(0, L, 23)]))
        ref, ref_abs = oracle.indexer_scores(to_np(d["q_idx"])[rows], to_np(d["w"])[rows],
                                             to_np(d["k_idx"]), rows + 1, with_abs=True)
        check_scores(to_np(scores[torch.as_tensor(rows, device=DEV)]), ref, ref_abs, what="8k rows")


# ---------------------------------------------------------------------------------------
# topk_select: same fp32 scores on both sides -> the sets must be identical
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols,k,ties,causal,per_row", [
    (7, 50, 5, True, False, False),
    (33, 300, 64, True, True, False),
    (16, 5000, 2048, False, False, True),
    (4, 70000, 2048, True, False, False),
    (9, 20000, 8192, False, False, True),
    (5, 1000, 1000, False, False, False),
])
def test_topk_select_exact(rows, cols, k, ties, causal, per_row):
    say(f"topk_select rows={rows} cols={cols} k={k} ties={ties} causal={causal} per_row={per_row}")
    r = np.random.default_rng(rows * 1000 + cols)
    if ties:
        sc = r.integers(-5, 6, size=(rows, cols)).astype(np.float32)
        sc[sc == 0] = -0.0 if r.random() < 0.5 else 0.0
    else:
        sc = r.standard_normal((rows, cols)).astype(np.float32)
    valid = None if causal else r.integers(1, cols + 1, size=rows).astype(np.int32)
    if valid is not None:
        valid[0] = cols
    kpr = r.integers(1, k + 1, size=rows).astype(np.int32) if per_row else None
    with sa.Handle(sa.Config(max_topk=max(k, 1))) as h:
        st = torch.from_numpy(sc).to(DEV)
        idx = torch.full((rows, k), -7, device=DEV, dtype=torch.int32)
        sa.topk_select(h, st, k, idx, valid_len=None if valid is None else torch.from_numpy(valid).to(DEV),
                       k_per_row=None if kpr is None else torch.from_numpy(kpr).to(DEV))
        assert sa.sparse_attn_check(h) == 0
        gi = to_np(idx)
    vis = np.minimum(np.arange(rows) + 1, cols) if valid is None else valid
    ref = oracle.topk(sc.astype(np.float64), vis, k, k_per_row=kpr)
    for i in range(rows):
        got = gi[i][gi[i] >= 0]
        exp = ref[i][ref[i] >= 0]
        assert np.array_equal(np.sort(got), np.sort(exp)), f"row {i}"
        assert np.all(np.diff(got) > 0), "indices must be ascending"
        assert np.all(gi[i][len(got):] == -1)


# ---------------------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("topk", [32, 256])
def test_prefill_tiny(topk):
    wl = inputs.WORKLOADS["tiny_prefill"]
    say(f"prefill tiny_prefill L=256 topk={topk}")
    d = inputs.prefill_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl, max_topk=256)) as h:
        out, lse, idx = _prefill(h, d, topk)
    _check_prefill_rows(d, out, lse, idx, topk, np.arange(256), latent=False, d_v=64,
                        what=f"tiny k={topk}")
    if topk >= 256:  # every row selects all visible tokens: dense causal attention
        ref = oracle.prefill(to_np(d["q"]), to_np(d["k"]), to_np(d["v"]), to_np(d["q_idx"]),
                             to_np(d["w"]), to_np(d["k_idx"]), top_k=256)
        assert np.abs(to_np(out) - ref["out"]).max() <= 2e-3


@pytest.mark.parametrize("L,topk", [(200, 64), (333, 128), (700, 512)])
def test_prefill_latent_small(L, topk):
    wl = inputs.WORKLOADS["prefill_8k"]
    say(f"prefill latent L={L} topk={topk}")
    d = inputs.prefill_inputs(wl, DEV, L=L, seed=L)
    with sa.Handle(inputs.library_config(wl, max_topk=topk)) as h:
        out, lse, idx = _prefill(h, d, topk)
    _check_prefill_rows(d, out, lse, idx, topk, np.arange(L), latent=True, d_v=512,
                        what=f"latent L={L} k={topk}")


def test_prefill_latent_dense_when_k_covers_all():
    wl = inputs.WORKLOADS["prefill_8k"]
    L = 130
    say(f"prefill latent dense L={L} topk={L}")
    d = inputs.prefill_inputs(wl, DEV, L=L, seed=99)
    with sa.Handle(inputs.library_config(wl, max_topk=L)) as h:
        out, lse, idx = _prefill(h, d, L)
    gi = to_np(idx)
    for t in range(L):
        assert np.array_equal(gi[t][:t + 1], np.arange(t + 1)) and np.all(gi[t][t + 1:] == -1)
    ref = oracle.prefill(to_np(d["q"]), to_np(d["k"]), None, to_np(d["q_idx"]), to_np(d["w"]),
                         to_np(d["k_idx"]), top_k=L, d_v=512)
    check_attention(to_np(out), to_np(lse), ref["out"], ref["lse"], what="dense latent")


def test_prefill_8k_sampled():
    wl = inputs.WORKLOADS["prefill_8k"]
    say("prefill prefill_8k L=8192 topk=2048 (sampled rows)")
    d = inputs.prefill_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _prefill(h, d, wl.topk)
        out2, lse2, idx2 = _prefill(h, d, wl.topk)
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2), "not deterministic"
    rows = np.unique(np.concatenate([[0, 1, 2, 100, 2046, 2047, 2048, 2049, 4000, 8190, 8191],
                                     np.random.default_rng(8).integers(0, wl.L, 37)]))
    _check_prefill_rows(d, out, lse, idx, wl.topk, rows, latent=True, d_v=512, what="8k")


@pytest.mark.parametrize("L,topk", [(2051, 256), (4100, 2048)])
def test_prefill_latent_ragged(L, topk):
    """Several 8-row tiles and 64-key tiles with ragged tails; rows below and above k."""
    wl = inputs.WORKLOADS["prefill_8k"]
    say(f"prefill latent ragged L={L} topk={topk}")
    d = inputs.prefill_inputs(wl, DEV, L=L, seed=L + 1)
    with sa.Handle(inputs.library_config(wl, max_topk=topk)) as h:
        out, lse, idx = _prefill(h, d, topk)
        out2, lse2, idx2 = _prefill(h, d, topk)
    # the persistent kernel takes tiles in whatever order workgroups arrive; results must not
    # depend on it
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2), "not deterministic"
    rows = np.unique(np.concatenate([np.arange(0, 9), [topk - 2, topk - 1, topk, topk + 1],
                                     np.arange(L - 9, L),
                                     np.random.default_rng(L).integers(0, L, 24)]))
    _check_prefill_rows(d, out, lse, idx, topk, rows, latent=True, d_v=512, what=f"ragged L={L}")


def test_prefill_all_scores_tied():
    """q_idx = 0 makes every score exactly 0: the selection is the lowest k indices.  Rows
    past 8192 keys have more tied candidates than the on-chip buffer holds."""
    wl = inputs.WORKLOADS["prefill_8k"]
    L, topk = 8300, 512
    say(f"prefill all-tied scores L={L} topk={topk}")
    d = inputs.prefill_inputs(wl, DEV, L=L, seed=77)
    d["q_idx"] = torch.zeros_like(d["q_idx"])
    with sa.Handle(inputs.library_config(wl, max_topk=topk)) as h:
        out, lse, idx = _prefill(h, d, topk)
    gi = to_np(idx)
    for t in (0, 5, topk - 1, topk, 4000, 8191, 8192, 8250, L - 1):
        m = min(topk, t + 1)
        assert np.array_equal(gi[t][:m], np.arange(m)), f"row {t}"
        assert np.all(gi[t][m:] == -1)
    rows = np.array([0, topk, 8192, L - 1])
    _check_prefill_rows(d, out, lse, idx, topk, rows, latent=True, d_v=512, what="all-tied")


def test_prefill_128k_sampled():
    """The 131072-token prefill exactly as the benchmark runs it, checked on 256 rows: the first 64, the
    last 64, the rows right after 32 salient positions (spread over the sequence) and 96 drawn at random."""
    wl = inputs.WORKLOADS["prefill_128k"]
    say(f"prefill prefill_128k L={wl.L} topk={wl.topk} (256 sampled rows)")
    d = inputs.prefill_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _prefill(h, d, wl.topk)
    sal = np.sort(d["salient"])
    after = sal[np.linspace(0, len(sal) - 1, 32).astype(np.int64)] + 1
    after = after[after < wl.L]
    rng = np.random.default_rng(128)
    fixed = np.unique(np.concatenate([np.arange(64), np.arange(wl.L - 64, wl.L), after]))
    pool = np.setdiff1d(np.arange(wl.L), fixed)
    rows = np.unique(np.concatenate([fixed, rng.choice(pool, 256 - len(fixed), replace=False)]))
    assert len(rows) == 256
    _check_prefill_rows(d, out, lse, idx, wl.topk, rows, latent=True, d_v=512, what="128k")
    del out, lse, idx, d
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------------------
def _decode(h, d, ws=None):
    B = d["q"].shape[0]
    s = h.cfg
    out = torch.empty((B, s.n_heads, s.d_v), device=DEV, dtype=torch.float32)
    lse = torch.empty((B, s.n_heads), device=DEV, dtype=torch.float32)
    idx = torch.empty((B, s.max_topk), device=DEV, dtype=torch.int32)
    ws = sa.workspace(h, sa.SA_OP_DECODE, B, d["max_ctx"]) if ws is None else ws
    sa.sparse_attn_decode(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], d["v_pages"], d["kidx_pages"],
                          d["block_table"], d["ctx_len"], d["topk"], d["max_ctx"], out, lse, idx, ws)
    assert sa.sparse_attn_check(h) == 0
    return out, lse, idx


def _check_decode(d, out, lse, idx, seqs, d_v, what, latent=True):
    seqs = np.asarray(seqs)
    table = to_np(d["block_table"])[seqs]
    ctx = d["ctx_np"][seqs]
    kv_pool, tab = compact_pages(d["kv_pages"], table, ctx)
    ki_pool, _ = compact_pages(d["kidx_pages"], table, ctx)
    v_pool = None if latent else compact_pages(d["v_pages"], table, ctx)[0]
    topk = to_np(d["topk"])[seqs]
    gi = to_np(idx)
    diffs = 0
    sel = np.full((len(seqs), gi.shape[1]), -1, dtype=np.int32)
    for i, b in enumerate(seqs):
        n = int(ctx[i])
        kI = oracle.depage(ki_pool, tab[i], n)
        sc = oracle.indexer_scores(to_np(d["q_idx"])[b:b + 1], to_np(d["w"])[b:b + 1], kI, [n])[0]
        diffs += check_topk_row(gi[b], sc, min(int(topk[i]), n), n, what=f"{what} seq {b}")
        sel[i] = gi[b]
    res = oracle.decode(to_np(d["q"])[seqs], to_np(d["q_idx"])[seqs], to_np(d["w"])[seqs], kv_pool,
                        v_pool, ki_pool, tab, ctx, top_k=topk, k_max=gi.shape[1], d_v=d_v)
    # attention on the GPU's own selection
    ref_out = np.empty_like(res["out"])
    ref_lse = np.empty_like(res["lse"])
    for i in range(len(seqs)):
        n = int(ctx[i])
        Kb = oracle.depage(kv_pool, tab[i], n)
        Vb = None if latent else oracle.depage(v_pool, tab[i], n)
        o, l = oracle.attention_rows(to_np(d["q"])[seqs[i]:seqs[i] + 1], Kb, Vb, sel[i:i + 1],
                                     oracle.default_scale(d["q"].shape[-1]), d_v=d_v)
        ref_out[i], ref_lse[i] = o[0], l[0]
    err = check_attention(to_np(out)[seqs], to_np(lse)[seqs], ref_out, ref_lse, what=what)
    say(f"{what}: seqs={len(seqs)} near-tie set diffs={diffs} max|dO|={err:.2e}")


def _check_decode_light(d, out, lse, idx, seqs, what):
    """_check_decode for long contexts, moving to the host only each checked sequence's index keys and its
    selected latent rows: the oracle's scores over every cached token decide the top-k check, and the
    oracle's attention runs on the GPU's own selection (rows gathered through the block table)."""
    P = d["kidx_pages"].shape[1]
    gi = to_np(idx)
    topk = to_np(d["topk"])
    diffs, err = 0, 0.0
    for b in np.asarray(seqs):
        n = int(d["ctx_np"][b])
        m = min(int(topk[b]), n)
        pages = d["block_table"][b, :(n + P - 1) // P].long()
        kI = to_np(d["kidx_pages"][pages].reshape(-1, d["kidx_pages"].shape[-1])[:n])
        sc = oracle.indexer_scores(to_np(d["q_idx"])[b:b + 1], to_np(d["w"])[b:b + 1], kI, [n])[0]
        diffs += check_topk_row(gi[b], sc, m, n, what=f"{what} seq {b}")
        sel = torch.as_tensor(gi[b][:m].astype(np.int64), device=DEV)
        rows = to_np(d["kv_pages"][pages[sel // P], sel % P].reshape(m, 1, -1))
        o, l = oracle.attention_rows(to_np(d["q"])[b:b + 1], rows, None, np.arange(m)[None, :],
                                     oracle.default_scale(d["q"].shape[-1]), d_v=512)
        err = max(err, check_attention(to_np(out)[b:b + 1], to_np(lse)[b:b + 1], o, l, what=f"{what} seq {b}"))
    say(f"{what}: seqs={len(seqs)} near-tie set diffs={diffs} max|dO|={err:.2e}")


def test_decode_small_paged():
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [1, 63, 64, 65, 300, 1000, 2500, 129]
    say(f"decode latent small ctx={ctx} topk=256")
    d = inputs.decode_inputs(inputs.small(wl, topk=256), DEV, ctx=ctx, seed=3)
    with sa.Handle(inputs.library_config(wl, max_topk=256)) as h:
        out, lse, idx = _decode(h, d)
    _check_decode(d, out, lse, idx, np.arange(len(ctx)), 512, "decode small")


def test_decode_generic_paged():
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], shapes=inputs.TINY, topk=16)
    ctx = [1, 5, 64, 100, 333]
    say(f"decode tiny (fp32, generic kernels) ctx={ctx} topk=16")
    d = inputs.decode_inputs(wl, DEV, ctx=ctx, seed=4)
    with sa.Handle(inputs.library_config(wl, max_topk=16)) as h:
        out, lse, idx = _decode(h, d)
    _check_decode(d, out, lse, idx, np.arange(len(ctx)), 64, "decode tiny", latent=False)


def test_decode_b64_sampled():
    wl = inputs.WORKLOADS["decode_b64"]
    say("decode decode_b64 B=64 ctx U[16K,64K] topk=2048 (8 sequences checked)")
    d = inputs.decode_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _decode(h, d)
        out2, lse2, idx2 = _decode(h, d)
    assert torch.equal(out, out2) and torch.equal(idx, idx2), "not deterministic"
    seqs = [0, 1, int(np.argmax(d["ctx_np"])), int(np.argmin(d["ctx_np"])), 17, 33, 50, 63]
    _check_decode(d, out, lse, idx, sorted(set(seqs)), 512, "decode_b64")


def test_decode_b64_128k_sampled():
    """The decode step exactly as the benchmark runs it (64 sequences at 131072 tokens)."""
    wl = inputs.WORKLOADS["decode_b64_128k"]
    say("decode decode_b64_128k B=64 ctx=131072 topk=2048 (16 sequences checked)")
    d = inputs.decode_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _decode(h, d)
    _check_decode_light(d, out, lse, idx, np.arange(0, 64, 4), "decode_b64_128k")
    del out, lse, idx, d
    torch.cuda.empty_cache()


def test_decode_all_scores_tied():
    """q_idx = 0 makes every score exactly 0: each sequence selects its lowest k_b tokens.  The
    long sequences have more tied candidates than the on-chip buffer holds."""
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [5, 300, 2049, 9000, 20000]
    say(f"decode all-tied scores ctx={ctx} topk=2048")
    d = inputs.decode_inputs(inputs.small(wl, topk=2048), DEV, ctx=ctx, seed=9)
    d["q_idx"] = torch.zeros_like(d["q_idx"])
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _decode(h, d)
    gi = to_np(idx)
    for b, n in enumerate(ctx):
        m = min(2048, n)
        assert np.array_equal(gi[b][:m], np.arange(m)), f"seq {b}"
        assert np.all(gi[b][m:] == -1)
    _check_decode(d, out, lse, idx, np.arange(len(ctx)), 512, "decode all-tied")


def test_decode_rl_sweep_every_step():
    """The RL-rollout sweep as the benchmark runs it: caches generated once for 32768 tokens per sequence,
    one decode step of all 256 sequences at each n = 1024 i (i = 1..32) with the per-sequence budgets
    min(n, max(256, floor(rho n))); 16 sequences checked at every step (a different 16 each time)."""
    wl = inputs.WORKLOADS["decode_rl_sweep"]
    n_max = wl.ctx_range[1]
    say(f"decode decode_rl_sweep B={wl.B}, all 32 steps n = 1024..{n_max} (16 sequences checked per step)")
    d = inputs.decode_inputs(wl, DEV, ctx=np.full(wl.B, n_max))
    with sa.Handle(inputs.library_config(wl, max_topk=8192)) as h:
        ws = sa.workspace(h, sa.SA_OP_DECODE, wl.B, n_max)
        for i, n in enumerate(range(1024, n_max + 1, 1024)):
            k = inputs.rl_budget(n, d["rho"])
            step = dict(d)
            step["topk"] = torch.from_numpy(k.astype(np.int32)).to(DEV)
            step["ctx_len"] = torch.full((wl.B,), n, dtype=torch.int32, device=DEV)
            step["ctx_np"] = np.full(wl.B, n)
            step["max_ctx"] = n
            out, lse, idx = _decode(h, step, ws)
            seqs = (np.arange(16) * 16 + i) % wl.B
            _check_decode_light(step, out, lse, idx, seqs, f"rl n={n}")


def test_decode_1024_row_ranges_at_boundaries():
    """64 sequences with budgets up to 8192 spread their selected rows over more workgroups than two
    rounds of the CUs take, so the decode attention runs 1024-row ranges; budgets and contexts sit on
    and around the range and chunk boundaries (1, 32, 1023..1025, 2047, 2049, 8192)."""
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], topk=8192)
    base_ctx = [1, 33, 1024, 1025, 2047, 3000, 8192, 9000]
    base_k = [1, 32, 1023, 1025, 2047, 2049, 8192, 8192]
    ctx = np.array([base_ctx[b % 8] for b in range(64)])
    k = np.array([base_k[(b + b // 8) % 8] for b in range(64)])
    say(f"decode 1024-row ranges B=64 max_topk=8192 ctx={base_ctx} k={base_k}")
    d = inputs.decode_inputs(wl, DEV, ctx=ctx, seed=21)
    d["topk"] = torch.from_numpy(k.astype(np.int32)).to(DEV)
    with sa.Handle(inputs.library_config(wl, max_topk=8192)) as h:
        out, lse, idx = _decode(h, d)
    gi = to_np(idx)
    for b in range(64):
        m = min(int(k[b]), int(ctx[b]))
        assert np.all(gi[b][:m] >= 0) and np.all(gi[b][m:] == -1), f"seq {b}: {m} selected slots"
    # one sequence per distinct (context, budget) pair
    seqs = sorted({(int(c), int(kb)): b for b, (c, kb) in enumerate(zip(ctx, k))}.values())
    _check_decode(d, out, lse, idx, seqs, 512, "decode 1024-row ranges")


def test_decode_sixteen_512_row_ranges():
    """Few sequences with budgets up to 8192: 512-row ranges, up to 16 partial states merged per head."""
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], topk=8192)
    ctx = np.array([9000, 8192, 8193, 5000])
    k = np.array([8192, 8192, 7681, 4097])
    say(f"decode 512-row ranges B=4 max_topk=8192 ctx={ctx.tolist()} k={k.tolist()}")
    d = inputs.decode_inputs(wl, DEV, ctx=ctx, seed=22)
    d["topk"] = torch.from_numpy(k.astype(np.int32)).to(DEV)
    with sa.Handle(inputs.library_config(wl, max_topk=8192)) as h:
        out, lse, idx = _decode(h, d)
    _check_decode(d, out, lse, idx, np.arange(4), 512, "decode 16 ranges")


# ---------------------------------------------------------------------------------------
# error paths that need a device
# ---------------------------------------------------------------------------------------
def test_host_validation_errors():
    say("host validation errors")
    wl = inputs.WORKLOADS["prefill_8k"]
    d = inputs.prefill_inputs(wl, DEV, L=64)
    with sa.Handle(inputs.library_config(wl, max_topk=32)) as h:
        out = torch.empty((64, 16, 512), device=DEV)
        small_ws = torch.empty(16, dtype=torch.uint8, device=DEV)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_prefill(h, d["q"], d["k"], None, d["q_idx"], d["w"], d["k_idx"], 32, out, ws=small_ws)
        assert e.value.status == sa.SA_ERR_WORKSPACE
        ws = sa.workspace(h, sa.SA_OP_PREFILL, 64)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_prefill(h, d["q"], d["k"], None, d["q_idx"], d["w"], d["k_idx"], 33, out, ws=ws)
        assert e.value.status == sa.SA_ERR_INVALID_ARG and "topk" in str(e.value)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_prefill(h, d["q"], d["k"], d["k"], d["q_idx"], d["w"], d["k_idx"], 8, out, ws=ws)
        assert e.value.status == sa.SA_ERR_INVALID_ARG
        big_q = torch.empty((16385, 64, 128), dtype=torch.bfloat16, device=DEV)
        tiny = torch.empty(1, device=DEV)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.indexer_scores(h, big_q, tiny, big_q, tiny)
        assert e.value.status == sa.SA_ERR_UNSUPPORTED
        torch.cuda.synchronize()


def test_device_checks_flag_bad_block_table():
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [200, 100]
    say("decode with a corrupted block table entry and an out-of-range ctx_len")
    d = inputs.decode_inputs(inputs.small(wl, topk=64), DEV, ctx=ctx, seed=5)
    bt = d["block_table"].clone()
    bt[0, 1] = 10 ** 6     # beyond the pool
    d["block_table"] = bt
    cl = d["ctx_len"].clone()
    cl[1] = d["max_ctx"] + 1  # beyond max_ctx
    d["ctx_len"] = cl
    with sa.Handle(inputs.library_config(wl, max_topk=64)) as h:
        B = 2
        out = torch.empty((B, 16, 512), device=DEV)
        ws = sa.workspace(h, sa.SA_OP_DECODE, B, d["max_ctx"])
        sa.sparse_attn_decode(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], None, d["kidx_pages"],
                              d["block_table"], d["ctx_len"], d["topk"], d["max_ctx"], out, ws=ws)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_check(h)
        assert e.value.status == sa.SA_ERR_DEVICE_CHECK
        assert sa.sparse_attn_check(h) == 0  # cleared
        assert torch.isfinite(out).all()


@pytest.mark.gpu
def test_decode_selected_tokens_on_a_bad_page_get_no_weight():
    """k >= n selects every visible token, including the 64 whose block-table entry is corrupted: the
    entry is flagged and those tokens get no weight, so the output equals attention over the others
    (two 512-row ranges and a partial last chunk for the longer sequence)."""
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [300, 700]
    say(f"decode, k >= n, bad block-table entry selected ctx={ctx}")
    d = inputs.decode_inputs(inputs.small(wl, topk=1024), DEV, ctx=ctx, seed=13)
    good = to_np(d["block_table"]).copy()
    bt = d["block_table"].clone()
    bt[0, 2] = 10 ** 6  # tokens 128..191 of sequence 0
    d["block_table"] = bt
    with sa.Handle(inputs.library_config(wl, max_topk=1024)) as h:
        B = len(ctx)
        out = torch.empty((B, 16, 512), device=DEV)
        lse = torch.empty((B, 16), device=DEV)
        idx = torch.empty((B, 1024), device=DEV, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_DECODE, B, d["max_ctx"])
        sa.sparse_attn_decode(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], None, d["kidx_pages"],
                              d["block_table"], d["ctx_len"], d["topk"], d["max_ctx"], out, lse, idx, ws)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_check(h)
        assert e.value.status == sa.SA_ERR_DEVICE_CHECK
    gi = to_np(idx)
    for b, n in enumerate(ctx):
        assert np.array_equal(gi[b][:n], np.arange(n)) and np.all(gi[b][n:] == -1), f"seq {b}"
    kv_pool, tab = compact_pages(d["kv_pages"], good, np.asarray(ctx))
    ref_out = np.empty((B, 16, 512))
    ref_lse = np.empty((B, 16))
    for b, n in enumerate(ctx):
        keep = np.arange(n) if b else np.concatenate([np.arange(128), np.arange(192, n)])
        sel = np.full((1, 1024), -1, dtype=np.int32)
        sel[0, :len(keep)] = keep
        K = oracle.depage(kv_pool, tab[b], n)
        o, l = oracle.attention_rows(to_np(d["q"])[b:b + 1], K, None, sel, oracle.default_scale(576), d_v=512)
        ref_out[b], ref_lse[b] = o[0], l[0]
    err = check_attention(to_np(out), to_np(lse), ref_out, ref_lse, what="bad page selected")
    say(f"bad page selected: max|dO|={err:.2e}")
