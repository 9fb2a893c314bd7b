"""Pins for the oracle's per-query top-k (CPU only).

Page: "Sparse Attention and RL Optimization: Three Technical Breakthroughs in LLM
Post-Training", section 2.3 (top-k preceding tokens per query by index score) and the
section 2.5 pseudocode (score.topk(top_k)).  Ties go to the lower index."""
import json
import os

import numpy as np

import oracle


def test_hand_worked_ties(golden_dir):
    with open(os.path.join(golden_dir, "topk_ties_example.json")) as f:
        g = json.load(f)
    sc = np.array(g["scores"], dtype=np.float64)
    for k, exp in g["expected"].items():
        got = oracle.topk(sc, [len(sc)], int(k))
        np.testing.assert_array_equal(got[0], np.array(exp))


def _brute_force_select(row, n, k):
    """Selected set by counting: s is selected iff fewer than min(k, n) visible keys rank
    strictly ahead of it (higher score, or equal score and lower index)."""
    m = min(k, n)
    sel = set()
    for s in range(n):
        ahead = 0
        for u in range(n):
            if row[u] > row[s] or (row[u] == row[s] and u < s):
                ahead += 1
        if ahead < m:
            sel.add(s)
    return sel


def test_matches_brute_force_ranking_with_many_ties():
    r = np.random.default_rng(11)
    for trial in range(30):
        n_cols = int(r.integers(1, 40))
        rows = int(r.integers(1, 6))
        sc = r.integers(-3, 4, size=(rows, n_cols)).astype(np.float64)  # heavy ties
        vis = r.integers(1, n_cols + 1, size=rows)
        k = int(r.integers(1, n_cols + 3))
        idx = oracle.topk(sc, vis, k)
        for i in range(rows):
            got = [int(x) for x in idx[i] if x >= 0]
            assert len(got) == len(set(got)) == min(k, vis[i])
            assert set(got) == _brute_force_select(sc[i], int(vis[i]), k)
            assert np.all(idx[i][len(got):] == -1)


def test_invariants_random_real_scores():
    r = np.random.default_rng(12)
    n = 300
    sc = r.standard_normal((4, n))
    sc[:, ::7] = 0.0  # exact ties at zero, as ReLU scores produce
    vis = np.array([1, 17, 150, 300])
    prev = None
    for k in (1, 5, 64, 150, 299, 300, 400):
        idx = oracle.topk(sc, vis, k)
        for i in range(4):
            sel = [int(x) for x in idx[i] if x >= 0]
            assert len(sel) == min(k, vis[i])
            assert all(0 <= s < vis[i] for s in sel)
            if len(sel) < vis[i]:
                rest = np.setdiff1d(np.arange(vis[i]), sel)
                assert sc[i, sel].min() >= sc[i, rest].max()
            if k >= vis[i]:
                assert sorted(sel) == list(range(vis[i]))
            if prev is not None:
                assert set(prev[i]) <= set(sel)  # nested in k
        prev = [[int(x) for x in row if x >= 0] for row in idx]


def test_per_row_budget():
    sc = np.arange(10, dtype=np.float64)[None, :].repeat(3, 0)
    idx = oracle.topk(sc, [10, 10, 4], 6, k_per_row=[2, 6, 6])
    np.testing.assert_array_equal(idx[0], [9, 8, -1, -1, -1, -1])
    np.testing.assert_array_equal(idx[1], [9, 8, 7, 6, 5, 4])
    np.testing.assert_array_equal(idx[2], [3, 2, 1, 0, -1, -1])
