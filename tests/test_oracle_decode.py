"""Pins for the oracle's paged decode (CPU only).

Page: "Long-Context LLMs Explained: Sparse Attention, Stable Reinforcement Learning, and
Verifiable Synthetic Data", section 2.3: at each decode step only the selected k KV
entries are read, composed with paged KV management; k may grow slowly with length."""
import numpy as np

import oracle


def _seq(seed, n, H=4, d_qk=24, d_v=16, H_I=2, d_I=8):
    r = np.random.default_rng(seed)
    return dict(q=r.standard_normal((n, H, d_qk)).astype(np.float32),
                K=r.standard_normal((n, 1, d_qk)).astype(np.float32),
                q_idx=r.standard_normal((n, H_I, d_I)).astype(np.float32),
                w=r.standard_normal((n, H_I)).astype(np.float32),
                k_idx=r.standard_normal((n, d_I)).astype(np.float32))


def _page(arr, page, table, n_pages):
    pool = np.zeros((n_pages, page) + arr.shape[1:], arr.dtype)
    for s in range(arr.shape[0]):
        pool[table[s // page], s % page] = arr[s]
    return pool


def test_depage_layout():
    pool = np.arange(3 * 4).reshape(3, 4)  # 3 pages of 4 slots
    np.testing.assert_array_equal(oracle.depage(pool, [2, 0], 6), [8, 9, 10, 11, 0, 1])


def test_paged_decode_equals_last_prefill_row_for_any_block_table():
    page, d_v = 4, 16
    seqs = [_seq(31, 37), _seq(32, 9)]
    n_pages = sum((s["q"].shape[0] + page - 1) // page for s in seqs) + 3
    r = np.random.default_rng(33)
    for shuffled in (False, True):
        perm = r.permutation(n_pages) if shuffled else np.arange(n_pages)
        tables = np.full((2, 16), -1, np.int32)
        used = 0
        pools = {"K": [], "k_idx": []}
        for b, s in enumerate(seqs):
            nb = (s["q"].shape[0] + page - 1) // page
            tables[b, :nb] = perm[used:used + nb]
            used += nb
        kv_pool = np.zeros((n_pages, page, 1, 24), np.float32)
        ki_pool = np.zeros((n_pages, page, 8), np.float32)
        for b, s in enumerate(seqs):
            kv_pool += _page(s["K"], page, tables[b], n_pages)
            ki_pool += _page(s["k_idx"], page, tables[b], n_pages)
        q = np.stack([s["q"][-1] for s in seqs])
        qi = np.stack([s["q_idx"][-1] for s in seqs])
        w = np.stack([s["w"][-1] for s in seqs])
        ctx = np.array([s["q"].shape[0] for s in seqs])
        dec = oracle.decode(q, qi, w, kv_pool, None, ki_pool, tables, ctx, top_k=[5, 3],
                            k_max=5, d_v=d_v)
        for b, s in enumerate(seqs):
            n = s["q"].shape[0]
            pre = oracle.prefill(s["q"], s["K"], None, s["q_idx"], s["w"], s["k_idx"],
                                 top_k=[5, 3][b], rows=[n - 1], d_v=d_v)
            got = [x for x in dec["idx"][b] if x >= 0]
            np.testing.assert_array_equal(got, [x for x in pre["idx"][0] if x >= 0])
            np.testing.assert_array_equal(dec["out"][b], pre["out"][0])
            np.testing.assert_array_equal(dec["lse"][b], pre["lse"][0])


def test_budget_closed_form():
    assert oracle.decode_budget(1024, 0.05) == 256     # floor(51.2) < 256
    assert oracle.decode_budget(32768, 0.25) == 8192
    assert oracle.decode_budget(100, 0.1) == 100       # never more than the context
    assert oracle.decode_budget(20480, 0.2) == 4096
    assert oracle.decode_budget(3000, 0.0999) == 299   # floor, not round


def test_paged_rows_equal_the_contiguous_prefill_of_each_sequence():
    """prefill_paged over every position of two paged sequences, rows shuffled and interleaved,
    equals the plain causal prefill of each sequence laid out contiguously, row for row."""
    page, d_v, k = 4, 16, 6
    seqs = [_seq(41, 23), _seq(42, 14)]
    n_pages = sum((s["q"].shape[0] + page - 1) // page for s in seqs) + 2
    perm = np.random.default_rng(43).permutation(n_pages)
    tables = np.full((2, 8), -1, np.int32)
    used = 0
    for b, s in enumerate(seqs):
        nb = (s["q"].shape[0] + page - 1) // page
        tables[b, :nb] = perm[used:used + nb]
        used += nb
    kv_pool = np.zeros((n_pages, page, 1, 24), np.float32)
    ki_pool = np.zeros((n_pages, page, 8), np.float32)
    for b, s in enumerate(seqs):
        kv_pool += _page(s["K"], page, tables[b], n_pages)
        ki_pool += _page(s["k_idx"], page, tables[b], n_pages)
    row_seq = np.concatenate([np.full(s["q"].shape[0], b) for b, s in enumerate(seqs)])
    row_pos = np.concatenate([np.arange(s["q"].shape[0]) for s in seqs])
    order = np.random.default_rng(44).permutation(len(row_seq))
    row_seq, row_pos = row_seq[order], row_pos[order]
    q = np.stack([seqs[b]["q"][p] for b, p in zip(row_seq, row_pos)])
    qi = np.stack([seqs[b]["q_idx"][p] for b, p in zip(row_seq, row_pos)])
    w = np.stack([seqs[b]["w"][p] for b, p in zip(row_seq, row_pos)])
    res = oracle.prefill_paged(q, qi, w, kv_pool, None, ki_pool, tables, row_seq, row_pos, k, d_v=d_v)
    pre = [oracle.prefill(s["q"], s["K"], None, s["q_idx"], s["w"], s["k_idx"], top_k=k, d_v=d_v) for s in seqs]
    for t, (b, p) in enumerate(zip(row_seq, row_pos)):
        np.testing.assert_array_equal(res["idx"][t], pre[b]["idx"][p])
        np.testing.assert_array_equal(res["out"][t], pre[b]["out"][p])
        np.testing.assert_array_equal(res["lse"][t], pre[b]["lse"][p])
