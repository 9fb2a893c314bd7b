"""Pins for the oracle's two-tier (block -> token) selection (CPU only).

Page: "A Guide to Sparse Attention and Efficient Reinforcement Learning in LLM Long-Context
Inference", section 1.1: the history is cut into fixed-size blocks, a few blocks are kept by
their indexer scores, and token-level selection runs inside the kept blocks.  Readings: a
block's score is its best visible token score; blocks and tokens both rank by (score desc,
index asc), the tie rule of "Sparse Attention and RL Optimization...", section 2.3."""
import json
import os

import numpy as np

import oracle


def _rank_ahead(vals, idxs, a, b):
    """True if element a ranks strictly ahead of element b (higher value, or equal value and
    lower index)."""
    return vals[a] > vals[b] or (vals[a] == vals[b] and idxs[a] < idxs[b])


def test_hand_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "block_topk_hand_example.json")) as f:
        g = json.load(f)
    sc = np.array(g["scores"], dtype=np.float64)
    for c in g["cases"]:
        idx, blocks = oracle.block_topk(sc, [c["visible"]], len(c["idx"]), g["block_size"],
                                        c["n_blocks"], with_blocks=True)
        np.testing.assert_array_equal(idx[0], c["idx"])
        np.testing.assert_array_equal(blocks[0], c["blocks"])


def _tie_heavy(r, rows, n):
    return r.integers(-3, 4, size=(rows, n)).astype(np.float64)


def test_all_blocks_kept_equals_flat_topk():
    """Keeping every block leaves every visible token a candidate: flat top-k."""
    r = np.random.default_rng(21)
    for _ in range(40):
        n = int(r.integers(1, 90))
        rows = int(r.integers(1, 5))
        sc = _tie_heavy(r, rows, n)
        vis = r.integers(1, n + 1, size=rows)
        bs = int(r.choice([1, 2, 3, 4, 8, 16]))
        k = int(r.integers(1, n + 3))
        nb = -(-n // bs) + int(r.integers(0, 3))
        np.testing.assert_array_equal(oracle.block_topk(sc, vis, k, bs, nb), oracle.topk(sc, vis, k))


def test_at_least_k_blocks_kept_equals_flat_topk():
    """With n_blocks >= k the kept blocks always contain the flat top-k tokens: each of them
    lies in a block whose best score is at least the k-th score, and a block that holds none of
    them ranks behind every block that does (ties included, by the lower-index rule)."""
    r = np.random.default_rng(22)
    for _ in range(60):
        n = int(r.integers(1, 120))
        rows = int(r.integers(1, 5))
        sc = _tie_heavy(r, rows, n)
        vis = r.integers(1, n + 1, size=rows)
        bs = int(r.choice([2, 4, 5, 8]))
        k = int(r.integers(1, 12))
        nb = k + int(r.integers(0, 3))
        np.testing.assert_array_equal(oracle.block_topk(sc, vis, k, bs, nb), oracle.topk(sc, vis, k))


def test_unit_blocks_equal_flat_topk_of_the_smaller_budget():
    """Blocks of one token: the kept blocks are the flat top-n_blocks tokens."""
    r = np.random.default_rng(23)
    for _ in range(40):
        n = int(r.integers(1, 60))
        sc = _tie_heavy(r, 3, n)
        vis = r.integers(1, n + 1, size=3)
        k = int(r.integers(1, 20))
        nb = int(r.integers(1, 20))
        got = oracle.block_topk(sc, vis, k, 1, nb)
        ref = oracle.topk(sc, vis, min(k, nb))
        np.testing.assert_array_equal(got[:, :min(k, nb)], ref)
        assert np.all(got[:, min(k, nb):] == -1)


def test_small_budget_takes_whole_blocks():
    """n_blocks * block_size <= k: every visible token of the kept blocks is selected, and the
    kept blocks are the flat top-n_blocks of the block maxima (numpy's reduceat)."""
    r = np.random.default_rng(24)
    for _ in range(40):
        n = int(r.integers(1, 100))
        bs = int(r.choice([2, 4, 8]))
        nb = int(r.integers(1, 6))
        k = nb * bs + int(r.integers(0, 4))
        row = r.standard_normal(n)
        row[r.random(n) < 0.3] = 0.0
        vis = int(r.integers(1, n + 1))
        bmax = np.maximum.reduceat(row[:vis], np.arange(0, vis, bs))
        kept = oracle.topk(bmax, [len(bmax)], min(nb, len(bmax)))[0]
        expect = sorted(s for s in range(vis) if s // bs in set(kept.tolist()))
        got = oracle.block_topk(row, [vis], k, bs, nb)[0]
        assert sorted(int(x) for x in got if x >= 0) == expect
        assert np.all(got[len(expect):] == -1)


def test_exchange_invariants_by_brute_force():
    """Every kept block ranks ahead of every dropped one; every selected token lies in a kept
    block and ranks ahead of every unselected candidate; the sizes are min(n_blocks, blocks) and
    min(k, candidates).  Checked pair by pair."""
    r = np.random.default_rng(25)
    for _ in range(40):
        n = int(r.integers(1, 70))
        bs = int(r.choice([1, 3, 4, 7]))
        row = _tie_heavy(r, 1, n)[0]
        vis = int(r.integers(1, n + 1))
        nb = int(r.integers(1, 8))
        k = int(r.integers(1, 25))
        idx, blocks = oracle.block_topk(row, [vis], k, bs, nb, with_blocks=True)
        n_blk = -(-vis // bs)
        kept = [int(b) for b in blocks[0] if b >= 0]
        assert len(kept) == len(set(kept)) == min(nb, n_blk)
        bmax = [max(row[s] for s in range(j * bs, min((j + 1) * bs, vis))) for j in range(n_blk)]
        blk_ids = list(range(n_blk))
        for a in kept:
            for b in set(blk_ids) - set(kept):
                assert _rank_ahead(bmax, blk_ids, a, b)
        cands = [s for s in range(vis) if s // bs in kept]
        sel = [int(x) for x in idx[0] if x >= 0]
        assert len(sel) == len(set(sel)) == min(k, len(cands))
        assert set(sel) <= set(cands)
        toks = list(range(n))
        for a in sel:
            for b in set(cands) - set(sel):
                assert _rank_ahead(row, toks, a, b)
        # rank order of the output
        for a, b in zip(sel, sel[1:]):
            assert _rank_ahead(row, toks, a, b)


def test_per_row_budget_and_padding():
    row = np.arange(12, dtype=np.float64)  # block 2 (tokens 8-11) is best, then 1, then 0
    sc = np.stack([row, row, row])
    idx = oracle.block_topk(sc, [12, 12, 6], 5, 4, 2, k_per_row=[2, 5, 5])
    np.testing.assert_array_equal(idx[0], [11, 10, -1, -1, -1])
    np.testing.assert_array_equal(idx[1], [11, 10, 9, 8, 7])
    np.testing.assert_array_equal(idx[2], [5, 4, 3, 2, 1])  # visible 6: blocks 1 (4-5) and 0


def test_pipeline_with_blocks_equals_attention_on_its_selection():
    """prefill(..., blocks=...) is the flat pipeline with the two-tier selection in place of
    top-k: it must equal attention over block_topk of its own scores, and with every block
    kept the flat pipeline."""
    r = np.random.default_rng(26)
    L, HI, dI, H, d = 40, 2, 8, 2, 16
    q_idx = r.standard_normal((L, HI, dI)).astype(np.float32)
    w = r.random((L, HI)).astype(np.float32)
    k_idx = r.standard_normal((L, dI)).astype(np.float32)
    q = r.standard_normal((L, H, d)).astype(np.float32)
    K = r.standard_normal((L, H, d)).astype(np.float32)
    V = r.standard_normal((L, H, d)).astype(np.float32)
    res = oracle.prefill(q, K, V, q_idx, w, k_idx, 6, blocks=(4, 2), with_scores=True)
    idx = oracle.block_topk(res["scores"], np.arange(1, L + 1), 6, 4, 2)
    np.testing.assert_array_equal(res["idx"], idx)
    out, _ = oracle.attention_rows(q, K, V, idx, oracle.default_scale(d))
    np.testing.assert_array_equal(res["out"], out)
    full = oracle.prefill(q, K, V, q_idx, w, k_idx, 6, blocks=(4, 10))
    flat = oracle.prefill(q, K, V, q_idx, w, k_idx, 6)
    np.testing.assert_array_equal(full["idx"], flat["idx"])


def test_parity_checker_accepts_the_oracle_and_rejects_planted_mistakes():
    """The GPU tests' two-tier checker (tests/parity.py) passes the oracle's own selection and
    fails a selection with a planted mistake: a token swapped for an unselected candidate, a
    kept block swapped for a dropped one, a duplicate."""
    import pytest

    from tests.parity import check_block_topk_row
    r = np.random.default_rng(27)
    row = r.standard_normal(500)
    idx = oracle.block_topk(row, [500], 40, 16, 4)[0]
    assert check_block_topk_row(np.sort(idx), row, 500, 40, 16, 4) == 0
    sel = set(int(x) for x in idx)
    _, kept = oracle.block_topk(row, [500], 40, 16, 4, with_blocks=True)
    kept = set(int(b) for b in kept[0])
    cands = [s for s in range(500) if s // 16 in kept and s not in sel]
    swapped = np.sort(np.array(sorted(sel - {int(idx[-1])}) + [cands[0]]))
    with pytest.raises(AssertionError):
        check_block_topk_row(swapped, row, 500, 40, 16, 4)
    outside = [s for s in range(500) if s // 16 not in kept]
    moved = np.sort(np.array(sorted(sel - {int(idx[0])}) + [outside[0]]))
    with pytest.raises(AssertionError):
        check_block_topk_row(moved, row, 500, 40, 16, 4)
    dup = np.sort(idx.copy())
    dup[1] = dup[0]
    with pytest.raises(AssertionError):
        check_block_topk_row(dup, row, 500, 40, 16, 4)
