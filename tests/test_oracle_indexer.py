"""Pins for the oracle's indexer score (CPU only).

Page: "Sparse Attention and RL Optimization: Three Technical Breakthroughs in LLM
Post-Training", section 2.2 (I(t,s) = sum_j w(t,j) ReLU(q(t,j).k(s)); ReLU terms are
non-negative) and section 2.5 (single-head pseudocode relu(i_q @ i_k.T), causal mask)."""
import json
import os

import numpy as np

import oracle


def _load_golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        g = json.load(f)

    def conv(x):
        return np.array([[float(v) for v in row] for row in x])
    return g, conv


def test_hand_worked_example(golden_dir):
    g, conv = _load_golden(golden_dir, "indexer_hand_example.json")
    q = np.array(g["q_idx"], dtype=np.float32)
    w = np.array(g["w"], dtype=np.float32)
    k = np.array(g["k_idx"], dtype=np.float32)
    sc, ab = oracle.indexer_scores(q, w, k, [1, 2, 3], with_abs=True)
    np.testing.assert_array_equal(sc, conv(g["scores"]))
    np.testing.assert_array_equal(ab, conv(g["abs_scores"]))
    np.testing.assert_array_equal(oracle.topk(sc, [1, 2, 3], 1), np.array(g["top1"]))
    np.testing.assert_array_equal(oracle.topk(sc, [1, 2, 3], 2), np.array(g["top2"]))


def _rand(seed, L=24, H_I=3, d_I=8, w_low=-1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((L, H_I, d_I)).astype(np.float32)
    k = r.standard_normal((L, d_I)).astype(np.float32)
    w = r.uniform(w_low, 1.0, (L, H_I)).astype(np.float32)
    return q, w, k


def test_single_head_unit_weight_is_relu_of_gemm():
    # [P1] 2.5 pseudocode: score = relu(i_q @ i_k.T), then causal mask.
    q, _, k = _rand(1, L=33, H_I=1, d_I=16)
    L = q.shape[0]
    sc = oracle.indexer_scores(q, np.ones((L, 1), np.float32), k, np.arange(1, L + 1))
    ref = np.maximum(q[:, 0, :].astype(np.float64) @ k.astype(np.float64).T, 0.0)
    ref[np.triu_indices(L, 1)] = -np.inf
    np.testing.assert_allclose(sc, ref, rtol=1e-12, atol=1e-12)


def test_causal_mask_only_looks_back():
    q, w, k = _rand(2)
    L = q.shape[0]
    sc = oracle.indexer_scores(q, w, k, np.arange(1, L + 1))
    t, s = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    assert np.all(np.isneginf(sc[s > t]))
    assert np.all(np.isfinite(sc[s <= t]))


def test_heads_sum_and_linear_in_w():
    q, w, k = _rand(3)
    L, H_I, _ = q.shape
    vis = np.arange(1, L + 1)
    full = oracle.indexer_scores(q, w, k, vis)
    per_head = [oracle.indexer_scores(q[:, j:j + 1], w[:, j:j + 1], k, vis) for j in range(H_I)]
    fin = np.isfinite(full)
    np.testing.assert_allclose(full[fin], sum(p[fin] for p in per_head), rtol=1e-12, atol=1e-12)
    w2 = _rand(4)[1]
    a = oracle.indexer_scores(q, w, k, vis)
    b = oracle.indexer_scores(q, w2, k, vis)
    c = oracle.indexer_scores(q, w + w2, k, vis)
    np.testing.assert_allclose(c[fin], a[fin] + b[fin], rtol=1e-6, atol=1e-6)


def test_positive_homogeneity_in_keys():
    # Scaling a key by a power of two scales every ReLU term exactly.
    q, w, k = _rand(5)
    L = q.shape[0]
    vis = np.arange(1, L + 1)
    base = oracle.indexer_scores(q, w, k, vis)
    k4 = k.copy()
    k4[7] *= 4.0
    scaled = oracle.indexer_scores(q, w, k4, vis)
    np.testing.assert_array_equal(scaled[:, 7], 4.0 * base[:, 7])
    np.testing.assert_array_equal(np.delete(scaled, 7, 1), np.delete(base, 7, 1))


def test_relu_terms_non_negative():
    # [P1] 2.2: ReLU gives non-negative terms; with w >= 0 every score is >= 0 and equals
    # the absolute-term sum; in general |I| <= A.
    q, w, k = _rand(6, w_low=0.0)
    L = q.shape[0]
    vis = np.arange(1, L + 1)
    sc, ab = oracle.indexer_scores(q, w, k, vis, with_abs=True)
    fin = np.isfinite(sc)
    assert np.all(sc[fin] >= 0.0)
    np.testing.assert_array_equal(sc[fin], ab[fin])
    q, w, k = _rand(7)
    sc, ab = oracle.indexer_scores(q, w, k, vis, with_abs=True)
    fin = np.isfinite(sc)
    assert np.all(np.abs(sc[fin]) <= ab[fin] * (1 + 1e-12))
    assert np.any(sc[fin] < 0.0)


def test_decode_visibility_row():
    # a single query seeing all n keys (decode) equals the last prefill row
    q, w, k = _rand(8)
    L = q.shape[0]
    pre = oracle.indexer_scores(q, w, k, np.arange(1, L + 1))
    dec = oracle.indexer_scores(q[-1:], w[-1:], k, [L])
    np.testing.assert_array_equal(dec[0], pre[-1])
