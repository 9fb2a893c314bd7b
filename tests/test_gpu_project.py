"""GPU parity of the index projections against the oracle (bf16 handle, latent shapes).

A bf16 output must be the round-to-nearest-even bf16 of a value within the fp32 accumulation
error of the exact projection: |gpu - exact| <= ulp(gpu) / 2 + 1e-5 * sum|terms|.  An fp32
output (w) must be within 1e-5 * sum|terms| of the exact value.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import indexer_selected_sparse_scores_amd as sa
import oracle
from indexer_selected_sparse_scores_amd import inputs
from tests.parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
ACC = 1e-5  # fp32 accumulation, relative to the sum of |terms|


def say(msg):
    print(msg, flush=True)


def _bf16(shape, std, gen):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16)


def _check_bf16(gpu, x, W, what):
    gpu = to_np(gpu).astype(np.float64)
    ref = oracle.project(to_np(x), to_np(W))
    ab = oracle.project_abs(to_np(x), to_np(W))
    ulp = np.where(gpu != 0, np.exp2(np.floor(np.log2(np.abs(gpu) + 1e-300)) - 7), 0.0)
    err = np.abs(gpu - ref) - (0.5 * ulp + ACC * ab + 1e-30)
    bad = np.argwhere(err > 0)
    assert bad.size == 0, f"{what}: {len(bad)} outputs off, first {bad[0]}: gpu {gpu[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"
    say(f"{what}: max |gpu - exact| / sum|terms| = {np.max(np.abs(gpu - ref) / (ab + 1e-30)):.2e}")


def _check_f32(gpu, x, W, what):
    gpu = to_np(gpu).astype(np.float64)
    ref = oracle.project(to_np(x), to_np(W))
    ab = oracle.project_abs(to_np(x), to_np(W))
    assert np.all(np.abs(gpu - ref) <= ACC * ab + 1e-30), f"{what}: max rel {np.max(np.abs(gpu - ref) / (ab + 1e-30)):.2e}"


def _handle():
    return sa.Handle(inputs.library_config(inputs.WORKLOADS["decode_b64"]))


def test_project_q_ragged():
    g = torch.Generator().manual_seed(21)
    L, K = 300, 16 * 576
    say(f"indexer_project_q L={L}")
    q = _bf16((L, 16, 576), 1.0, g).to(DEV)
    W_iq = _bf16((64 * 128, K), K ** -0.5, g).to(DEV)
    W_w = _bf16((64, K), K ** -0.5, g).to(DEV)
    with _handle() as h:
        q_idx = torch.empty((L, 64, 128), dtype=torch.bfloat16, device=DEV)
        w = torch.empty((L, 64), dtype=torch.float32, device=DEV)
        sa.indexer_project_q(h, q, W_iq, W_w, q_idx, w)
        # the two halves alone give the same results
        q_idx2 = torch.empty_like(q_idx)
        w2 = torch.empty_like(w)
        sa.indexer_project_q(h, q, W_iq, None, q_idx2, None)
        sa.indexer_project_q(h, q, None, W_w, None, w2)
        assert sa.sparse_attn_check(h) == 0
    x = q.reshape(L, K)
    _check_bf16(q_idx.reshape(L, -1), x, W_iq, "q_idx")
    _check_f32(w, x, W_w, "w")
    assert torch.equal(q_idx, q_idx2) and torch.equal(w, w2)


@pytest.mark.parametrize("H,d_qk,H_I,d_I,L", [
    (1, 64, 2, 128, 1),       # one K block, one column tile, one row
    (8, 192, 32, 64, 257),    # a ragged row tail past one 256-row tile
    (4, 128, 256, 32, 70),    # H_I = 256: the weight tile is full
    (16, 576, 48, 128, 513),  # H_I * d_I = 6144: 24 column tiles, the last row tile ragged
])
def test_project_q_shapes(H, d_qk, H_I, d_I, L):
    g = torch.Generator().manual_seed(26 + L)
    K, N1 = H * d_qk, H_I * d_I
    say(f"indexer_project_q H={H} d_qk={d_qk} H_I={H_I} d_I={d_I} L={L}")
    q = _bf16((L, K), 1.0, g).to(DEV)
    W_iq = _bf16((N1, K), K ** -0.5, g).to(DEV)
    W_w = _bf16((H_I, K), K ** -0.5, g).to(DEV)
    cfg = sa.Config(n_idx_heads=H_I, d_idx=d_I, n_heads=H, d_qk=d_qk, d_v=min(d_qk, 512))
    with sa.Handle(cfg) as h:
        # sentinel rows past the end: the kernel writes none of them
        q_idx = torch.full((L + 3, N1), -9.0, dtype=torch.bfloat16, device=DEV)
        w = torch.full((L + 3, H_I), -9.0, dtype=torch.float32, device=DEV)
        sa.indexer_project_q(h, q, W_iq, W_w, q_idx, w)
        assert sa.sparse_attn_check(h) == 0
    _check_bf16(q_idx[:L], q, W_iq, "q_idx")
    _check_f32(w[:L], q, W_w, "w")
    assert torch.all(q_idx[L:] == -9.0) and torch.all(w[L:] == -9.0)


def test_project_k_contiguous_ragged():
    g = torch.Generator().manual_seed(22)
    L = 300
    say(f"indexer_project_k contiguous L={L}")
    k = _bf16((L, 576), 1.0, g).to(DEV)
    W_ik = _bf16((128, 576), 576 ** -0.5, g).to(DEV)
    with _handle() as h:
        k_idx = torch.empty((L, 128), dtype=torch.bfloat16, device=DEV)
        sa.indexer_project_k(h, k, W_ik, k_idx)
        assert sa.sparse_attn_check(h) == 0
    _check_bf16(k_idx, k, W_ik, "k_idx")


def _pool(n_pages, gen):
    sentinel = torch.full((n_pages, 64, 128), -7.0, dtype=torch.bfloat16)
    return sentinel.to(DEV)


def test_project_k_paged_prefill_from_mid_page():
    """One sequence, positions 100 .. 299 (starting inside its second page), shuffled pages: every
    row lands in its slot and no other slot is touched."""
    g = torch.Generator().manual_seed(23)
    L, pos0, n_pages = 200, 100, 12
    say(f"indexer_project_k paged prefill pos0={pos0} L={L}")
    k = _bf16((L, 576), 1.0, g).to(DEV)
    W_ik = _bf16((128, 576), 576 ** -0.5, g).to(DEV)
    table = torch.from_numpy(np.random.default_rng(23).permutation(n_pages)[:6].astype(np.int32)).reshape(1, 6)
    pool = _pool(n_pages, g)
    with _handle() as h:
        sa.indexer_project_k(h, k, W_ik, pool, block_table=table.to(DEV), n_pages=n_pages, pos0=pos0)
        assert sa.sparse_attn_check(h) == 0
    pool_np = to_np(pool)
    written = np.zeros((n_pages, 64), dtype=bool)
    rows = np.empty((L, 128))
    for t in range(L):
        page, slot = oracle.paged_slot(table.numpy(), 0, pos0 + t, 64, n_pages)
        rows[t] = pool_np[page, slot]
        written[page, slot] = True
    _check_bf16(torch.from_numpy(rows), k, W_ik, "paged k_idx")
    assert np.all(pool_np[~written] == -7.0), "a slot outside the written positions changed"


def test_project_k_paged_decode_rows_with_a_bad_entry():
    """A decode step: one new token per sequence at position ctx_len - 1; sequence 2's entry for
    that position is corrupted, so its row is skipped and the entry is flagged."""
    g = torch.Generator().manual_seed(24)
    B, n_pages, max_blocks = 5, 20, 4
    say(f"indexer_project_k decode rows B={B}")
    k = _bf16((B, 576), 1.0, g).to(DEV)
    W_ik = _bf16((128, 576), 576 ** -0.5, g).to(DEV)
    table = np.random.default_rng(24).permutation(n_pages)[:B * max_blocks].astype(np.int32).reshape(B, max_blocks)
    ctx = np.array([1, 64, 65, 200, 256], dtype=np.int32)
    table[2, (ctx[2] - 1) // 64] = n_pages + 3
    pool = _pool(n_pages, g)
    with _handle() as h:
        sa.indexer_project_k(h, k, W_ik, pool, block_table=torch.from_numpy(table).to(DEV), n_pages=n_pages,
                             row_seq=torch.arange(B, dtype=torch.int32, device=DEV),
                             row_pos=torch.from_numpy(ctx - 1).to(DEV))
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_check(h)
        assert e.value.status == sa.SA_ERR_DEVICE_CHECK
    pool_np = to_np(pool)
    ref = np.asarray([oracle.paged_slot(table, b, int(ctx[b]) - 1, 64, n_pages) for b in range(B)], dtype=object)
    assert ref[2] is None
    good = [b for b in range(B) if ref[b] is not None]
    rows = np.stack([pool_np[ref[b][0], ref[b][1]] for b in good])
    _check_bf16(torch.from_numpy(rows), k[good], W_ik, "decode k_idx")
    n_written = sum(1 for b in good)
    assert np.sum(np.any(pool_np != -7.0, axis=-1)) == n_written, "a slot other than the new tokens' changed"


def test_project_q_128k_sampled_rows():
    """The full query projection of the 128K prefill, checked on sampled rows."""
    g = torch.Generator(device=DEV).manual_seed(25)
    L, K = 131072, 16 * 576
    say(f"indexer_project_q L={L} (sampled rows)")
    q = (torch.randn((L, K), generator=g, device=DEV)).to(torch.bfloat16)
    W_iq = (torch.randn((8192, K), generator=g, device=DEV) * K ** -0.5).to(torch.bfloat16)
    W_w = (torch.randn((64, K), generator=g, device=DEV) * K ** -0.5).to(torch.bfloat16)
    with _handle() as h:
        q_idx = torch.empty((L, 8192), dtype=torch.bfloat16, device=DEV)
        w = torch.empty((L, 64), dtype=torch.float32, device=DEV)
        sa.indexer_project_q(h, q, W_iq, W_w, q_idx, w)
        assert sa.sparse_attn_check(h) == 0
    rows = np.unique(np.concatenate([[0, 1, L - 2, L - 1], np.random.default_rng(25).integers(0, L, 12)]))
    r = torch.from_numpy(rows).to(DEV)
    _check_bf16(q_idx[r], q[r], W_iq, "q_idx 128k rows")
    _check_f32(w[r], q[r], W_w, "w 128k rows")
    del q, W_iq, q_idx
    torch.cuda.empty_cache()
