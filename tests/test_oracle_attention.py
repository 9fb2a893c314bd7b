"""Pins for the oracle's sparse attention (CPU only).

Pages: "Sparse Attention and RL Optimization: Three Technical Breakthroughs in LLM
Post-Training", section 2.5 (gather the selected rows, softmax(q k_sel^T / sqrt(d)) v_sel);
"Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and
Verifiable Synthetic Data", section 2.4 (same, with the logits step explicit).
The library routine used as a pin is torch's scaled_dot_product_attention in float64."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _sdpa(q, K, V, causal, scale):
    """q [n_q,H,d], K [n_k,H,d], V [n_k,H,dv] -> [n_q,H,dv] via torch (float64, CPU)."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)[None]
    Kt = torch.from_numpy(np.asarray(K, np.float64)).permute(1, 0, 2)[None]
    Vt = torch.from_numpy(np.asarray(V, np.float64)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _mk(seed, L, H, H_kv, d_qk, d_v, latent):
    r = np.random.default_rng(seed)
    q = r.standard_normal((L, H, d_qk)).astype(np.float32)
    K = r.standard_normal((L, H_kv, d_qk)).astype(np.float32)
    V = None if latent else r.standard_normal((L, H_kv, d_v)).astype(np.float32)
    return q, K, V


@pytest.mark.parametrize("latent", [False, True])
def test_k_at_least_t_equals_dense_causal(latent):
    L, H = 40, 4
    H_kv, d_qk, d_v = (1, 24, 16) if latent else (4, 12, 12)
    q, K, V = _mk(21, L, H, H_kv, d_qk, d_v, latent)
    r = np.random.default_rng(22)
    q_idx = r.standard_normal((L, 2, 8)).astype(np.float32)
    w = r.uniform(0, 1, (L, 2)).astype(np.float32)
    k_idx = r.standard_normal((L, 8)).astype(np.float32)
    res = oracle.prefill(q, K, V, q_idx, w, k_idx, top_k=L, d_v=d_v)
    Kf = np.repeat(K, H // H_kv, axis=1)
    Vf = np.repeat(K[:, :, :d_v] if latent else V, H // H_kv, axis=1)
    ref = _sdpa(q, Kf, Vf, causal=True, scale=1.0 / math.sqrt(d_qk))
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_equals_attention_on_gathered_rows():
    L, H, d = 30, 3, 10
    q, K, V = _mk(23, L, H, H, d, d, False)
    r = np.random.default_rng(24)
    sel = np.array([[3, 17, 5, 29, -1, 0]], dtype=np.int32)
    s = sel[0][sel[0] >= 0]
    out, lse = oracle.attention_rows(q[:1], K, V, sel, scale=0.37)
    ref = _sdpa(q[:1], K[s], V[s], causal=False, scale=0.37)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    logits = 0.37 * np.einsum("hc,shc->hs", q[0].astype(np.float64), K[s].astype(np.float64))
    np.testing.assert_allclose(lse[0], logsumexp(logits, axis=1), rtol=1e-12)


def test_first_token_is_its_own_value():
    # t = 0 sees only itself: softmax weight exactly 1, output exactly V[0].
    q, K, V = _mk(25, 5, 2, 2, 6, 6, False)
    out, lse = oracle.attention_rows(q[:1], K, V, np.array([[0, -1, -1]]), scale=0.5)
    np.testing.assert_array_equal(out[0], V[0].astype(np.float64))
    np.testing.assert_allclose(lse[0], 0.5 * np.sum(q[0].astype(np.float64) * K[0], axis=1))


def test_zero_query_gives_mean_of_selected_values():
    q, K, V = _mk(26, 12, 2, 2, 6, 5, False)
    q0 = np.zeros_like(q[:1])
    sel = np.array([[4, 1, 9]])
    out, lse = oracle.attention_rows(q0, K, V, sel, scale=1.0)
    np.testing.assert_allclose(out[0], V[[4, 1, 9]].astype(np.float64).mean(0), rtol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(3.0), rtol=1e-14)


def test_two_keys_closed_form():
    # logits ln 3 and 0 -> weights 3/4 and 1/4
    q = np.ones((1, 1, 1), np.float32)
    K = np.array([[[math.log(3.0)]], [[0.0]]], np.float32)
    V = np.array([[[4.0, -8.0]], [[0.0, 8.0]]], np.float32)
    out, lse = oracle.attention_rows(q, K, V, np.array([[0, 1]]), scale=1.0)
    l3 = float(np.float32(math.log(3.0)))
    wa = math.exp(l3) / (math.exp(l3) + 1.0)
    np.testing.assert_allclose(out[0, 0], [4 * wa, -8 * wa + 8 * (1 - wa)], rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(math.exp(l3) + 1.0), rtol=1e-14)


def test_permutation_invariance_and_padding():
    q, K, V = _mk(27, 20, 4, 1, 16, 8, True)
    a = np.array([[2, 11, 19, 5]])
    b = np.array([[-1, 19, 5, -1, 2, 11]])
    oa, la = oracle.attention_rows(q[:1], K, None, a, 0.25, d_v=8)
    ob, lb = oracle.attention_rows(q[:1], K, None, b, 0.25, d_v=8)
    np.testing.assert_allclose(oa, ob, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_weights_sum_to_one():
    # with V = 1 everywhere the output is exactly a sum of softmax weights
    q, K, _ = _mk(28, 50, 2, 2, 8, 3, False)
    V = np.ones((50, 2, 3), np.float32)
    out, _ = oracle.attention_rows(q[:1], K, V, np.arange(50)[None], 0.3)
    np.testing.assert_allclose(out, 1.0, rtol=1e-14)
