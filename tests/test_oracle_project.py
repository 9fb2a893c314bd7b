"""Pins of the oracle's index projections (CPU): a hand-worked example, brute force, closed-form
special cases, bf16 rounding against an independent converter, and the paged placement rule."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "project_hand_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_project_hand_example():
    g = _golden()
    for case in ("rect", "square"):
        c = g[case]
        np.testing.assert_array_equal(oracle.project(c["x"], c["W"]), np.asarray(c["y"], dtype=np.float64))


def test_project_brute_force_and_special_cases():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7))
    W = rng.standard_normal((4, 7))
    brute = np.array([[sum(W[o, c] * x[t, c] for c in range(7)) for o in range(4)] for t in range(5)])
    np.testing.assert_allclose(oracle.project(x, W), brute, rtol=1e-12, atol=1e-12)
    # W = [I | 0] copies the leading columns exactly
    eye = np.hstack([np.eye(4), np.zeros((4, 3))])
    np.testing.assert_array_equal(oracle.project(x, eye), x[:, :4])
    # linear in W and in x
    W2 = rng.standard_normal((4, 7))
    np.testing.assert_allclose(oracle.project(x, W + W2), oracle.project(x, W) + oracle.project(x, W2), atol=1e-12)
    x2 = rng.standard_normal((5, 7))
    np.testing.assert_allclose(oracle.project(2 * x - 3 * x2, W), 2 * oracle.project(x, W) - 3 * oracle.project(x2, W),
                               atol=1e-12)
    # the absolute-term sum bounds the value and equals it for non-negative inputs
    assert np.all(np.abs(oracle.project(x, W)) <= oracle.project_abs(x, W) + 1e-12)
    np.testing.assert_allclose(oracle.project_abs(np.abs(x), np.abs(W)), oracle.project(np.abs(x), np.abs(W)))


def test_round_bf16_hand_values_and_independent_converter():
    g = _golden()["bf16"]
    np.testing.assert_array_equal(oracle.round_bf16(g["in"]), g["out"])
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(v.astype(np.float64)), ref)


def test_paged_slot_hand_cases_and_brute_force():
    g = _golden()["paging"]
    for pos, want in g["cases"]:
        got = oracle.paged_slot(g["block_table"], 0, pos, g["page_size"], g["n_pages"])
        assert (got is None and want is None) or list(got) == want, (pos, got, want)
    rng = np.random.default_rng(5)
    P, n_pages = 8, 40
    table = rng.permutation(n_pages)[:3 * 5].reshape(3, 5).astype(np.int32)
    table[1, 4] = -1
    for seq in range(3):
        for pos in range(-2, 5 * P + 3):
            got = oracle.paged_slot(table, seq, pos, P, n_pages)
            if 0 <= pos < 5 * P and table[seq, pos // P] >= 0:
                # token pos is the (pos % P)-th row of the pool page holding its logical page
                assert got == (int(table[seq, pos // P]), pos % P)
            else:
                assert got is None
