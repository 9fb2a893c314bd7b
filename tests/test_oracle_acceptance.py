"""Pins for the oracle's acceptance rate and its per-bin lower-tail statistic (CPU only).

Page: "Sparrow: Sparse Rollout for Stable and Efficient Long-context RL of Large Language Models",
section 3.1: alpha = E_{x~Q}[min(p(x)/q(x), 1)] = sum_x min(p(x), q(x)) per token; the study uses
its 5-percentile per bin of 2K positions."""
import json
import os

import numpy as np

import oracle


def test_hand_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "acceptance_hand_example.json")) as f:
        g = json.load(f)
    for c in g["alpha_cases"]:
        a = oracle.acceptance_rate([c["logits_p"]], [c["logits_q"]])
        assert abs(a[0] - c["alpha"]) < 1e-12
    b = g["bins"]
    count, mean, pct = oracle.bin_percentiles(b["alpha"], b["pos"], b["bin_size"], b["n_bins"], b["percentile"])
    np.testing.assert_array_equal(count, b["count"])
    for got, exp in ((mean, b["mean"]), (pct, b["pct"])):
        for x, e in zip(got, exp):
            assert (np.isnan(x) and e is None) or abs(x - e) < 1e-12


def test_one_minus_total_variation():
    """sum_x min(p, q) = 1 - (1/2) sum_x |p - q|, a different formula of the same quantity."""
    r = np.random.default_rng(51)
    lp = r.standard_normal((20, 1000)) * 3
    lq = lp + r.standard_normal((20, 1000)) * r.uniform(0, 2, size=(20, 1))
    a = oracle.acceptance_rate(lp, lq)
    p = np.exp(lp) / np.exp(lp).sum(1, keepdims=True)
    q = np.exp(lq) / np.exp(lq).sum(1, keepdims=True)
    np.testing.assert_allclose(a, 1 - 0.5 * np.abs(p - q).sum(1), rtol=0, atol=1e-12)
    assert np.all((a >= 0) & (a <= 1 + 1e-12))


def test_symmetry_identity_shift_and_disjoint_support():
    r = np.random.default_rng(52)
    lp = r.standard_normal((8, 300))
    lq = r.standard_normal((8, 300))
    np.testing.assert_allclose(oracle.acceptance_rate(lp, lq), oracle.acceptance_rate(lq, lp), atol=1e-14)
    np.testing.assert_allclose(oracle.acceptance_rate(lp, lp), 1.0, atol=1e-12)
    # a constant added to a row of logits leaves its distribution unchanged
    np.testing.assert_allclose(oracle.acceptance_rate(lp + 7.5, lq - 3.0), oracle.acceptance_rate(lp, lq), atol=1e-12)
    # all mass on different tokens: nothing shared
    a = np.full((1, 50), -1e4)
    b = a.copy()
    a[0, 3] = 0.0
    b[0, 40] = 0.0
    assert oracle.acceptance_rate(a, b)[0] < 1e-12


def test_percentiles_equal_numpy():
    """The interpolated order statistic is numpy's default percentile; counts and means by bin."""
    r = np.random.default_rng(53)
    alpha = 1 - r.beta(0.3, 3, size=5000)
    pos = r.integers(0, 9 * 2048, size=5000)
    count, mean, pct = oracle.bin_percentiles(alpha, pos, 2048, 10, 5.0)
    for j in range(10):
        x = alpha[pos // 2048 == j]
        assert count[j] == len(x)
        if len(x) == 0:
            assert np.isnan(pct[j]) and np.isnan(mean[j])
            continue
        assert abs(pct[j] - np.percentile(x, 5.0)) < 1e-12
        assert abs(mean[j] - x.mean()) < 1e-12
    for q in (0.0, 50.0, 100.0):
        _, _, pq = oracle.bin_percentiles(alpha, pos, 2048, 1, q)
        x = alpha[pos // 2048 == 0]
        assert abs(pq[0] - {0.0: x.min(), 50.0: np.median(x), 100.0: x.max()}[q]) < 1e-12
