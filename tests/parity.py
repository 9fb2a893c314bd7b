"""Parity helpers shared by the GPU tests: compare the HIP path with the oracle.

Tolerances (bf16 inputs, fp32 accumulation):
  * indexer scores: |I_gpu - I_ref| <= 2e-3 * A + 1e-6, where A = sum_j |w| ReLU(q.k) is the
    sum of absolute terms (for w >= 0 this is plain 2e-3 relative); masked entries -inf.
  * top-k sets: bit-exact, except where the oracle's m-th and (m+1)-th scores are within
    1e-3 relative (a near-tie); then every index in the symmetric difference must score
    within 1e-3 relative of the oracle's m-th score.
  * attention outputs: within 2e-3 absolute of the oracle evaluated on the GPU's own
    selection (after the top-k check passed); LSE within 2e-3 absolute as well.
  * two-tier (block -> token) sets: bit-exact, except where the oracle's kept-block boundary
    (its last kept and first dropped block scores) or its token boundary (m-th and (m+1)-th
    candidate scores) is a near-tie at 1e-3 relative; then every index in the symmetric
    difference must be a near-tie of the token boundary or lie in a block whose score is a
    near-tie of the block boundary.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

SCORE_REL = 2e-3
TIE_REL = 1e-3
ATTN_ABS = 2e-3


def to_np(t) -> np.ndarray:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def check_scores(gpu: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    masked = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), masked), f"{what}: mask differs"
    fin = ~masked
    err = np.abs(gpu[fin] - ref[fin])
    bound = SCORE_REL * ref_abs[fin] + 1e-6
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} scores out of tolerance, worst err "
                           f"{err.max():.3g} (bound there {bound[np.argmax(err - bound)]:.3g})")


def check_topk_row(gpu_row, ref_scores: np.ndarray, m: int, visible: int, what=""):
    """gpu_row: the GPU's index list (any order, -1 padded); ref_scores: oracle scores of
    this query over its visible keys (float64)."""
    g = np.asarray(gpu_row)
    sel = g[g >= 0]
    assert len(sel) == m, f"{what}: {len(sel)} selected, expected {m}"
    assert len(np.unique(sel)) == m, f"{what}: duplicate indices"
    assert sel.min() >= 0 and sel.max() < visible, f"{what}: index out of the visible range"
    assert np.all(g[m:] == -1) if len(g) > m else True, f"{what}: padding is not -1"
    ref_idx = oracle.topk(ref_scores[None, :visible], [visible], m)[0]
    G, O = set(sel.tolist()), set(ref_idx.tolist())
    if G == O:
        return 0
    sc = ref_scores[:visible]
    order = np.lexsort((np.arange(visible), -sc))
    tau = sc[order[m - 1]]
    tau2 = sc[order[m]] if m < visible else -np.inf
    tie = abs(tau - tau2) <= TIE_REL * max(abs(tau), abs(tau2)) or tau == tau2
    assert tie, f"{what}: sets differ without a near-tie (tau={tau}, next={tau2})"
    for s in G ^ O:
        assert abs(sc[s] - tau) <= TIE_REL * max(abs(tau), abs(sc[s])) or sc[s] == tau, \
            f"{what}: index {s} (score {sc[s]}) is not a near-tie of {tau}"
    return len(G ^ O)


def _near(a, b):
    return a == b or abs(a - b) <= TIE_REL * max(abs(a), abs(b))


def check_block_topk_row(gpu_row, ref_scores: np.ndarray, visible: int, k: int, block_size: int,
                         n_blocks: int, what=""):
    """Two-tier selection of one row against the oracle's block_topk on the oracle's scores.
    Returns the size of the (near-tie) symmetric difference."""
    g = np.asarray(gpu_row)
    sel = g[g >= 0]
    sc = np.asarray(ref_scores[:visible], dtype=np.float64)
    ref, kept = oracle.block_topk(sc, [visible], len(g), block_size, n_blocks, k_per_row=[k],
                                  with_blocks=True)
    O = set(int(x) for x in ref[0] if x >= 0)
    assert len(np.unique(sel)) == len(sel), f"{what}: duplicate indices"
    assert len(sel) == 0 or (sel.min() >= 0 and sel.max() < visible), f"{what}: index out of range"
    G = set(sel.tolist())
    assert np.all(g[len(sel):] == -1), f"{what}: padding is not -1"
    if G == O:
        return 0
    n_blk = -(-visible // block_size)
    bmax = np.array([sc[j * block_size:(j + 1) * block_size].max() for j in range(n_blk)])
    kept = [int(b) for b in kept[0] if b >= 0]
    tau_b = bmax[kept[-1]]
    dropped = np.setdiff1d(np.arange(n_blk), kept)
    tau_b2 = bmax[dropped].max() if len(dropped) else -np.inf
    cands = np.array([s for s in range(visible) if s // block_size in set(kept)])
    order = cands[np.lexsort((cands, -sc[cands]))]
    m = len(O)
    tau = sc[order[m - 1]]
    tau2 = sc[order[m]] if m < len(order) else -np.inf
    block_tie, token_tie = _near(tau_b, tau_b2), _near(tau, tau2)
    assert block_tie or token_tie, (f"{what}: sets differ without a near-tie (blocks {tau_b} / {tau_b2}, "
                                    f"tokens {tau} / {tau2})")
    if not block_tie:
        assert len(G) == len(O), f"{what}: {len(G)} selected, expected {len(O)}"
    for s in G ^ O:
        ok = (token_tie and _near(sc[s], tau)) or (block_tie and _near(bmax[s // block_size], tau_b))
        assert ok, f"{what}: index {s} (score {sc[s]}) is not a near-tie of a selection boundary"
    return len(G ^ O)


def check_attention(gpu_out, gpu_lse, ref_out, ref_lse, what=""):
    go = np.asarray(gpu_out, dtype=np.float64)
    err = np.abs(go - ref_out)
    assert np.all(np.isfinite(go)), f"{what}: non-finite output"
    assert err.max() <= ATTN_ABS, f"{what}: attention max abs err {err.max():.3g}"
    if gpu_lse is not None:
        gl = np.asarray(gpu_lse, dtype=np.float64)
        e2 = np.abs(gl - ref_lse)
        assert e2.max() <= ATTN_ABS, f"{what}: lse max abs err {e2.max():.3g}"
    return float(err.max())


def compact_pages(pages: torch.Tensor, table_rows: np.ndarray, ctx: np.ndarray):
    """Copy to host only the pool pages the given sequences use; returns (pool, table)
    with the table renumbered into that smaller pool.  Pure data selection."""
    P = pages.shape[1]
    used = []
    new_table = np.full(table_rows.shape, -1, dtype=np.int64)
    for i in range(table_rows.shape[0]):
        nb = (int(ctx[i]) + P - 1) // P
        new_table[i, :nb] = np.arange(len(used), len(used) + nb)
        used.extend(table_rows[i, :nb].tolist())
    sub = pages[torch.as_tensor(np.asarray(used, dtype=np.int64), device=pages.device)]
    return to_np(sub).astype(np.float32), new_table
