"""GPU parity of the two-tier (block -> token) selection: topk_select_blocks,
sparse_attn_prefill_blocks and sparse_attn_decode_blocks against the CPU oracle.

Page: "A Guide to Sparse Attention and Efficient Reinforcement Learning in LLM Long-Context
Inference", section 1.1 (blocks kept by their indexer scores, then token-level selection inside
them).  On given fp32 scores both sides rank the same values, so the selection must be
bit-exact; through the pipelines the tolerances of tests/parity.py apply."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import indexer_selected_sparse_scores_amd as sa
import oracle
from indexer_selected_sparse_scores_amd import inputs
from tests.parity import check_attention, check_block_topk_row, compact_pages, to_np

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


def _sets(rows_idx):
    return [sorted(int(x) for x in r if x >= 0) for r in rows_idx]


# ---------------------------------------------------------------------------------------
# topk_select_blocks on given scores: bit-exact
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols,k,bs,nb,dist,mode", [
    (7, 300, 16, 4, 5, "ties", "causal"),
    (9, 1000, 64, 16, 8, "normal", "valid"),
    (5, 5000, 256, 64, 8, "normal", "causal"),       # k > kept tokens on some rows
    (6, 20000, 2048, 64, 64, "relu", "valid"),
    (4, 20000, 2048, 64, 256, "relu", "perrow"),     # 16384 candidates, the LDS maximum
    (3, 100000, 1024, 16, 512, "normal", "valid"),   # 6250 blocks
    (4, 3000, 100, 256, 3, "ties", "valid"),         # blocks wider than a wave
    (4, 3000, 100, 1024, 2, "normal", "causal"),
    (5, 700, 50, 1, 40, "ties", "perrow"),           # unit blocks: flat top-min(k, n_blocks)
    (3, 900, 900, 8, 2000, "ties", "valid"),         # more blocks asked for than exist
])
def test_topk_select_blocks_exact(rows, cols, k, bs, nb, dist, mode):
    say(f"topk_select_blocks rows={rows} cols={cols} k={k} block={bs} n_blocks={nb} {dist} {mode}")
    r = np.random.default_rng(rows * 1000 + cols + bs)
    if dist == "ties":
        sc = r.integers(-3, 4, size=(rows, cols)).astype(np.float32)
    elif dist == "relu":  # many exact zeros, as all-negative index heads give
        sc = np.maximum(r.standard_normal((rows, cols)), 0).astype(np.float32)
    else:
        sc = r.standard_normal((rows, cols)).astype(np.float32)
    if mode == "causal":  # no lengths given: valid(r) = min(r + 1, cols)
        vis = np.minimum(np.arange(rows) + 1, cols)
        valid = None
    else:
        vis = r.integers(1, cols + 1, size=rows)
        vis[0] = cols
        valid = torch.from_numpy(vis.astype(np.int32)).to(DEV)
    kpr = None
    kr = np.full(rows, k)
    if mode == "perrow":
        kr = r.integers(1, k + 1, size=rows)
        kpr = torch.from_numpy(kr.astype(np.int32)).to(DEV)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    with sa.Handle(sa.Config(dtype="f32", n_idx_heads=4, d_idx=32, n_heads=4, n_kv_heads=4, d_qk=64, d_v=64,
                             v_from_k=False, max_topk=max(k, 16))) as h:
        sa.topk_select_blocks(h, torch.from_numpy(sc).to(DEV), k, bs, nb, idx, valid_len=valid, k_per_row=kpr)
        assert sa.sparse_attn_check(h) == 0
    ref = oracle.block_topk(sc.astype(np.float64), vis, k, bs, nb, k_per_row=kr)
    gi = to_np(idx)
    for i in range(rows):
        exp = sorted(int(x) for x in ref[i] if x >= 0)
        got = gi[i]
        assert list(got[:len(exp)]) == exp, f"row {i}: selection differs"
        assert np.all(got[len(exp):] == -1), f"row {i}: padding"


def test_topk_select_blocks_all_tied_and_partial_last_block():
    """Every score equal: the lowest-index blocks win and, inside them, the lowest tokens; a
    visible length that cuts the last block keeps only its visible tokens."""
    say("topk_select_blocks all tied")
    rows, cols = 4, 1000
    sc = torch.zeros((rows, cols), dtype=torch.float32, device=DEV)
    vis = np.array([1000, 130, 65, 3])
    idx = torch.empty((rows, 200), dtype=torch.int32, device=DEV)
    with sa.Handle(sa.Config(max_topk=256)) as h:
        sa.topk_select_blocks(h, sc, 200, 64, 3, idx, valid_len=torch.from_numpy(vis.astype(np.int32)).to(DEV))
        assert sa.sparse_attn_check(h) == 0
    gi = to_np(idx)
    for i, n in enumerate(vis):
        m = min(200, n, 3 * 64)
        assert list(gi[i][:m]) == list(range(m)), f"row {i}"
        assert np.all(gi[i][m:] == -1)


def test_topk_select_blocks_validation():
    say("topk_select_blocks argument checks")
    sc = torch.zeros((2, 100), dtype=torch.float32, device=DEV)
    idx = torch.empty((2, 8), dtype=torch.int32, device=DEV)
    with sa.Handle(sa.Config(max_topk=256)) as h:
        for bs, nb, status in ((3, 4, sa.SA_ERR_INVALID_ARG), (0, 4, sa.SA_ERR_INVALID_ARG),
                               (2048, 1, sa.SA_ERR_INVALID_ARG), (64, 0, sa.SA_ERR_INVALID_ARG),
                               (64, 2049, sa.SA_ERR_INVALID_ARG), (64, 257, sa.SA_ERR_UNSUPPORTED)):
            with pytest.raises(sa.SparseAttnError) as e:
                sa.topk_select_blocks(h, sc, 8, bs, nb, idx)
            assert e.value.status == status, (bs, nb)
        big = torch.zeros((1, 16385), dtype=torch.float32, device=DEV)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.topk_select_blocks(h, big, 8, 1, 4, idx[:1])
        assert e.value.status == sa.SA_ERR_UNSUPPORTED
        sa.sparse_attn_check(h)


# ---------------------------------------------------------------------------------------
# prefill with two-tier selection
# ---------------------------------------------------------------------------------------
def _prefill_blocks(h, d, topk, bs, nb):
    L = d["q"].shape[0]
    s = h.cfg
    out = torch.empty((L, s.n_heads, s.d_v), device=DEV, dtype=torch.float32)
    lse = torch.empty((L, s.n_heads), device=DEV, dtype=torch.float32)
    idx = torch.empty((L, topk), device=DEV, dtype=torch.int32)
    ws = sa.workspace(h, sa.SA_OP_PREFILL_BLOCKS, L)
    sa.sparse_attn_prefill_blocks(h, d["q"], d["k"], d["v"], d["q_idx"], d["w"], d["k_idx"], topk, bs, nb, out,
                                  lse, idx, ws)
    assert sa.sparse_attn_check(h) == 0
    return out, lse, idx


def _check_prefill_blocks_rows(d, out, lse, idx, topk, bs, nb, rows, latent, d_v, what):
    rows = np.asarray(rows, dtype=np.int64)
    rt = torch.as_tensor(rows, device=d["q"].device)
    sub = lambda t: to_np(t[rt])
    sc = oracle.indexer_scores(sub(d["q_idx"]), sub(d["w"]), to_np(d["k_idx"]), rows + 1)
    gi = sub(idx)
    diffs = 0
    for i, t in enumerate(rows):
        diffs += check_block_topk_row(gi[i], sc[i], int(t) + 1, topk, bs, nb, what=f"{what} row {t}")
    ref_out, ref_lse = oracle.attention_rows(sub(d["q"]), to_np(d["k"]), None if latent else to_np(d["v"]), gi,
                                             oracle.default_scale(d["q"].shape[-1]), d_v=d_v)
    err = check_attention(sub(out), sub(lse), ref_out, ref_lse, what=what)
    say(f"{what}: rows={len(rows)} near-tie set diffs={diffs} max|dO|={err:.2e}")
    return diffs


@pytest.mark.parametrize("topk,bs,nb", [(32, 16, 4), (32, 8, 64), (64, 32, 1)])
def test_prefill_blocks_tiny(topk, bs, nb):
    wl = inputs.WORKLOADS["tiny_prefill"]
    say(f"prefill_blocks tiny L=256 fp32 topk={topk} block={bs} n_blocks={nb}")
    d = inputs.prefill_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl, max_topk=max(topk, 256))) as h:
        out, lse, idx = _prefill_blocks(h, d, topk, bs, nb)
    _check_prefill_blocks_rows(d, out, lse, idx, topk, bs, nb, np.arange(wl.L), latent=False, d_v=64,
                               what="prefill_blocks tiny")


def test_prefill_blocks_equals_flat_when_blocks_cover_k():
    """n_blocks >= k keeps every block that holds a flat top-k token: same result as the flat
    prefill, bit for bit (the attention kernels see the same index lists)."""
    wl = inputs.WORKLOADS["tiny_prefill"]
    say("prefill_blocks tiny with n_blocks >= topk against sparse_attn_prefill")
    d = inputs.prefill_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl, max_topk=256)) as h:
        out, lse, idx = _prefill_blocks(h, d, 32, 4, 32)
        L = wl.L
        out2 = torch.empty_like(out)
        idx2 = torch.empty_like(idx)
        ws = sa.workspace(h, sa.SA_OP_PREFILL, L)
        sa.sparse_attn_prefill(h, d["q"], d["k"], d["v"], d["q_idx"], d["w"], d["k_idx"], 32, out2, None, idx2, ws)
        assert sa.sparse_attn_check(h) == 0
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("L,topk,bs,nb", [(2051, 256, 64, 8), (4100, 2048, 64, 64)])
def test_prefill_blocks_latent(L, topk, bs, nb):
    wl = inputs.WORKLOADS["prefill_8k"]
    say(f"prefill_blocks latent bf16 L={L} topk={topk} block={bs} n_blocks={nb}")
    d = inputs.prefill_inputs(wl, DEV, L=L)
    with sa.Handle(inputs.library_config(wl, max_topk=topk)) as h:
        out, lse, idx = _prefill_blocks(h, d, topk, bs, nb)
    rows = np.unique(np.concatenate([np.arange(0, 80), [bs * nb - 1, bs * nb, L // 2, L - 2, L - 1],
                                     np.random.default_rng(L).integers(0, L, 24)]))
    _check_prefill_blocks_rows(d, out, lse, idx, topk, bs, nb, rows, latent=True, d_v=512,
                               what=f"prefill_blocks L={L}")


# ---------------------------------------------------------------------------------------
# decode with two-tier selection
# ---------------------------------------------------------------------------------------
def _decode_blocks(h, d, bs, nb):
    B = d["q"].shape[0]
    s = h.cfg
    out = torch.empty((B, s.n_heads, s.d_v), device=DEV, dtype=torch.float32)
    lse = torch.empty((B, s.n_heads), device=DEV, dtype=torch.float32)
    idx = torch.empty((B, s.max_topk), device=DEV, dtype=torch.int32)
    ws = sa.workspace(h, sa.SA_OP_DECODE_BLOCKS, B, d["max_ctx"])
    sa.sparse_attn_decode_blocks(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], d["v_pages"], d["kidx_pages"],
                                 d["block_table"], d["ctx_len"], d["topk"], d["max_ctx"], bs, nb, out, lse, idx, ws)
    assert sa.sparse_attn_check(h) == 0
    return out, lse, idx


def _check_decode_blocks(d, out, lse, idx, bs, nb, seqs, d_v, what, latent=True):
    seqs = np.asarray(seqs)
    table = to_np(d["block_table"])[seqs]
    ctx = d["ctx_np"][seqs]
    kv_pool, tab = compact_pages(d["kv_pages"], table, ctx)
    ki_pool, _ = compact_pages(d["kidx_pages"], table, ctx)
    v_pool = None if latent else compact_pages(d["v_pages"], table, ctx)[0]
    topk = to_np(d["topk"])[seqs]
    gi = to_np(idx)
    diffs = 0
    ref_out = np.empty((len(seqs), d["q"].shape[1], d_v))
    ref_lse = np.empty((len(seqs), d["q"].shape[1]))
    for i, b in enumerate(seqs):
        n = int(ctx[i])
        kI = oracle.depage(ki_pool, tab[i], n)
        sc = oracle.indexer_scores(to_np(d["q_idx"])[b:b + 1], to_np(d["w"])[b:b + 1], kI, [n])[0]
        diffs += check_block_topk_row(gi[b], sc, n, int(topk[i]), bs, nb, what=f"{what} seq {b}")
        Kb = oracle.depage(kv_pool, tab[i], n)
        Vb = None if latent else oracle.depage(v_pool, tab[i], n)
        o, l = oracle.attention_rows(to_np(d["q"])[b:b + 1], Kb, Vb, gi[b:b + 1],
                                     oracle.default_scale(d["q"].shape[-1]), d_v=d_v)
        ref_out[i], ref_lse[i] = o[0], l[0]
    err = check_attention(to_np(out)[seqs], to_np(lse)[seqs], ref_out, ref_lse, what=what)
    say(f"{what}: seqs={len(seqs)} near-tie set diffs={diffs} max|dO|={err:.2e}")


@pytest.mark.parametrize("bs,nb", [(64, 6), (256, 2), (128, 3), (32, 12), (1024, 1)])
def test_decode_blocks_small_paged(bs, nb):
    """Blocks of one page take the indexer's page maxima as they are, wider blocks combine them,
    narrower ones are scored from the scores themselves."""
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [1, 63, 64, 65, 300, 1000, 2500, 129, 1100, 4097]
    say(f"decode_blocks latent small ctx={ctx} topk=256 block={bs} n_blocks={nb}")
    d = inputs.decode_inputs(inputs.small(wl, topk=256), DEV, ctx=ctx, seed=3)
    with sa.Handle(inputs.library_config(wl, max_topk=256)) as h:
        out, lse, idx = _decode_blocks(h, d, bs, nb)
    _check_decode_blocks(d, out, lse, idx, bs, nb, np.arange(len(ctx)), 512, f"decode_blocks small b{bs}")


def test_decode_blocks_generic_paged():
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], shapes=inputs.TINY, topk=16)
    ctx = [1, 5, 64, 100, 333]
    say(f"decode_blocks tiny (fp32, generic kernels) ctx={ctx} topk=16 block=8 n_blocks=3")
    d = inputs.decode_inputs(wl, DEV, ctx=ctx, seed=4)
    with sa.Handle(inputs.library_config(wl, max_topk=16)) as h:
        out, lse, idx = _decode_blocks(h, d, 8, 3)
    _check_decode_blocks(d, out, lse, idx, 8, 3, np.arange(len(ctx)), 64, "decode_blocks tiny", latent=False)


def test_decode_blocks_b64_128k_sampled():
    """The two-tier decode step as the benchmark runs it: 64 sequences at 131072 tokens, blocks of
    one 64-token page, 64 blocks kept, top-2048 inside them."""
    wl = inputs.WORKLOADS["decode_b64_128k"]
    say("decode_blocks decode_b64_128k B=64 ctx=131072 topk=2048 block=64 n_blocks=64 (4 sequences checked)")
    d = inputs.decode_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _decode_blocks(h, d, 64, 64)
        out2, lse2, idx2 = _decode_blocks(h, d, 64, 64)
    assert torch.equal(out, out2) and torch.equal(idx, idx2), "not deterministic"
    _check_decode_blocks(d, out, lse, idx, 64, 64, [0, 21, 42, 63], 512, "decode_blocks 128k")
    del out, lse, idx, out2, lse2, idx2, d
    torch.cuda.empty_cache()


def test_decode_blocks_rl_sweep_budgets():
    """Per-sequence budgets k_b of the RL-rollout sweep with 32 blocks of 64 kept: k_b above
    2048 leaves the whole kept set selected."""
    wl = inputs.WORKLOADS["decode_rl_sweep"]
    n = 20480
    say(f"decode_blocks decode_rl_sweep B=256 n={n} per-sequence k, block=64 n_blocks=32 (5 checked)")
    d = inputs.decode_inputs(wl, DEV, ctx=np.full(wl.B, n))
    k = inputs.rl_budget(n, d["rho"])
    d["topk"] = torch.from_numpy(k.astype(np.int32)).to(DEV)
    with sa.Handle(inputs.library_config(wl, max_topk=8192)) as h:
        out, lse, idx = _decode_blocks(h, d, 64, 32)
    _check_decode_blocks(d, out, lse, idx, 64, 32, [0, int(np.argmax(k)), int(np.argmin(k)), 128, 255], 512,
                         "decode_blocks rl")


@pytest.mark.parametrize("L,topk,bs,nb", [(3000, 512, 128, 3), (3000, 256, 256, 2), (2500, 300, 1024, 1)])
def test_prefill_blocks_fused_wide_blocks(L, topk, bs, nb):
    """Blocks of several 64-key tiles: the fused first pass's tile keys are combined per block."""
    wl = inputs.WORKLOADS["prefill_8k"]
    say(f"prefill_blocks fused L={L} topk={topk} block={bs} n_blocks={nb}")
    d = inputs.prefill_inputs(wl, DEV, L=L, seed=77)
    with sa.Handle(inputs.library_config(wl, max_topk=topk)) as h:
        out, lse, idx = _prefill_blocks(h, d, topk, bs, nb)
    rows = np.unique(np.concatenate([np.arange(0, 40), [bs * nb - 1, bs * nb, bs * nb + 1, L // 2, L - 2, L - 1],
                                     np.random.default_rng(L + bs).integers(0, L, 24)]))
    _check_prefill_blocks_rows(d, out, lse, idx, topk, bs, nb, rows, latent=True, d_v=512,
                               what=f"prefill_blocks fused b{bs}")


def test_prefill_blocks_fused_equals_flat_when_blocks_cover_k():
    """n_blocks >= k: the kept blocks hold every flat winner and the second pass scores tokens exactly as
    the fused indexer does, so the two-tier prefill equals the flat prefill bit for bit (40 of 65 blocks
    kept here, so the block stage is not trivial)."""
    wl = inputs.WORKLOADS["prefill_8k"]
    L, topk = 4100, 32
    say(f"prefill_blocks fused (64-token blocks, 40 kept) vs sparse_attn_prefill, L={L}, topk={topk}")
    d = inputs.prefill_inputs(wl, DEV, L=L, seed=78)
    with sa.Handle(inputs.library_config(wl, max_topk=topk)) as h:
        out, lse, idx = _prefill_blocks(h, d, topk, 64, 40)
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        idx2 = torch.empty_like(idx)
        ws = sa.workspace(h, sa.SA_OP_PREFILL, L)
        sa.sparse_attn_prefill(h, d["q"], d["k"], None, d["q_idx"], d["w"], d["k_idx"], topk, out2, lse2, idx2, ws)
        assert sa.sparse_attn_check(h) == 0
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)


def test_prefill_blocks_128k_sampled():
    """The two-tier prefill as the benchmark runs it: L = 131072, blocks of 64, 64 kept, top-2048."""
    wl = inputs.WORKLOADS["prefill_128k"]
    say("prefill_blocks prefill_128k L=131072 topk=2048 block=64 n_blocks=64 (sampled rows)")
    d = inputs.prefill_inputs(wl, DEV)
    with sa.Handle(inputs.library_config(wl)) as h:
        out, lse, idx = _prefill_blocks(h, d, wl.topk, 64, 64)
    sal = d["salient"]
    rows = np.unique(np.concatenate([[0, 2047, 4095, 4096, 4097, 65535, wl.L - 2, wl.L - 1],
                                     sal[[0, len(sal) // 2, -1]] + 1,
                                     np.random.default_rng(129).integers(0, wl.L, 5)]))
    _check_prefill_blocks_rows(d, out, lse, idx, wl.topk, 64, 64, rows, latent=True, d_v=512,
                               what="prefill_blocks 128k")
    del out, lse, idx, d
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------
# the fused prefill kernel's own scores, at the score tolerance
# ---------------------------------------------------------------------------------------
def _key_to_float(keys: np.ndarray) -> np.ndarray:
    """Inverse of the library's order-preserving map of fp32 scores to uint32 (sign bit set for scores >= 0,
    all bits flipped for negative ones)."""
    k = keys.astype(np.uint32)
    u = np.where(k & np.uint32(0x80000000), k & np.uint32(0x7FFFFFFF), ~k)
    return u.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("L", [1500, 4100])
def test_fused_prefill_scores_at_the_score_tolerance(L):
    """The two-tier prefill's first pass is the fused prefill indexer in its block-key mode: the same MFMA
    tiles and epilogue as the per-query selection, keeping for each row and 64-key tile the order key of the
    row's best score there.  Read back from the documented workspace layout ([index lists | 256-byte counter |
    block keys [L, ceil(L / 64)] uint32]), they must equal the oracle's per-tile maxima within
    2e-3 * (largest |w| ReLU sum of the tile) -- a direct check of the fused kernel's scores."""
    wl = inputs.WORKLOADS["prefill_8k"]
    K, bs, nb = 64, 64, 1  # rows with more than 64 visible keys keep block keys
    say(f"fused prefill block keys L={L} (scores of the fused kernel vs the oracle)")
    d = inputs.prefill_inputs(wl, DEV, L=L, seed=L + 3)
    with sa.Handle(inputs.library_config(wl, max_topk=K)) as h:
        out = torch.empty((L, 16, 512), device=DEV)
        idx = torch.empty((L, K), device=DEV, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_PREFILL_BLOCKS, L)
        sa.sparse_attn_prefill_blocks(h, d["q"], d["k"], None, d["q_idx"], d["w"], d["k_idx"], K, bs, nb, out, None,
                                      idx, ws)
        assert sa.sparse_attn_check(h) == 0
        ld = (L + 63) // 64
        off = (L * K * 4 + 255) // 256 * 256 + 256
        keys = ws[off:off + L * ld * 4].view(torch.int32).view(L, ld)
        rng = np.random.default_rng(L)
        rows = np.unique(np.concatenate([[64, 65, 127, 128, L - 1], rng.integers(64, L, 19)]))
        got = _key_to_float(to_np(keys[torch.as_tensor(rows, device=DEV)]).view(np.uint32))
    ref, ref_abs = oracle.indexer_scores(to_np(d["q_idx"])[rows], to_np(d["w"])[rows], to_np(d["k_idx"]), rows + 1,
                                         with_abs=True)
    worst = 0.0
    for i, t in enumerate(rows):
        for j in range(t // 64 + 1):
            seg = slice(64 * j, min(64 * j + 64, t + 1))
            m_ref = ref[i, seg].max()
            bound = 2e-3 * ref_abs[i, seg].max() + 1e-6
            err = abs(got[i, j] - m_ref)
            worst = max(worst, err / bound)
            assert err <= bound, f"row {t} tile {j}: {got[i, j]} vs {m_ref} (bound {bound:.3g})"
    say(f"  {len(rows)} rows, every visible tile: worst error {worst:.3f} of the bound")
