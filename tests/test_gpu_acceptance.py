"""GPU parity of the acceptance rate and its per-bin statistics against the CPU oracle.

Page: "Sparrow: Sparse Rollout for Stable and Efficient Long-context RL of Large Language Models",
section 3.1 (alpha = sum_x min(p(x), q(x)) per token; its 5-percentile per bin of 2K positions).

Tolerance for alpha: 1e-4 absolute.  Both kernels sum in fp32: a thread adds at most about V/1024 terms
in sequence (149 at V = 151936; the single-read path 20 per lane) before tree and chunk reductions, so
each of the two normalisers and the sum of minima carries a relative error well below 1e-5, and exp2
with the log2(e) scaling adds a few 1e-7; alpha <= 1, so the total stays below 1e-4.  Every case runs
both paths: the two-pass kernel (no workspace) and the single-read one (a workspace; used where V % 4 == 0
and a token's rows fit 32 chunks of 3520 float4).  The percentile of a bin is 1-Lipschitz in
the largest change of any value, so it inherits the same bound; on given fp32 values it must equal
the oracle's up to the final rounding to fp32 (1 ulp)."""
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
ALPHA_ABS = 1e-4


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _handle():
    return sa.Handle(sa.Config())


def _alpha(h, lp, lq, V=None, once=False):
    T = lp.shape[0]
    alpha = torch.empty(T, dtype=torch.float32, device=DEV)
    ws = sa.workspace(h, sa.SA_OP_ACCEPT, T, lp.shape[1] if V is None else V) if once else None
    sa.acceptance_rate(h, lp, lq, alpha, V=V, ws=ws)
    assert sa.sparse_attn_check(h) == 0
    return to_np(alpha)


# (64, 151936): 11 chunks a token, 2 or 3 tokens per group of workgroups; (9, 151936, 8): padded rows, most
# groups idle; (1, 151936): one token, one group; (33, 40004, 4): 3 chunks, the last one shorter; (5, 4): one chunk of one float4; V % 4 != 0
# and V past 32 chunks take the two-pass kernel on both paths
@pytest.mark.parametrize("once", [False, True])
@pytest.mark.parametrize("T,V,pad", [(64, 151936, 0), (9, 151936, 8), (1, 151936, 0), (33, 40004, 4), (7, 1001, 3), (5, 4, 0),
                                     (3, 1, 0), (2, 4 * 3520 * 33, 0)])
def test_alpha_matches_oracle(T, V, pad, once):
    say(f"acceptance_rate T={T} V={V} row padding={pad} single-read={once}")
    d = inputs.acceptance_inputs(T, V + pad, DEV, seed=61)
    with _handle() as h:
        a = _alpha(h, d["logits_p"], d["logits_q"], V=V, once=once)
    ref = oracle.acceptance_rate(to_np(d["logits_p"])[:, :V], to_np(d["logits_q"])[:, :V])
    err = np.abs(a - ref).max()
    say(f"  max|d alpha|={err:.2e}, alpha range [{ref.min():.4f}, {ref.max():.4f}]")
    assert err <= ALPHA_ABS


def test_alpha_single_read_repeats_bit_for_bit():
    """The single-read path merges the chunks' normalisers and partial sums in chunk order: the same
    inputs give the same bits on every call, whichever workgroups publish first."""
    T, V = 96, 151936
    say(f"acceptance_rate single-read determinism T={T} V={V}")
    d = inputs.acceptance_inputs(T, V, DEV, seed=65)
    with _handle() as h:
        runs = [_alpha(h, d["logits_p"], d["logits_q"], once=True) for _ in range(3)]
    assert all(np.array_equal(runs[0], r) for r in runs[1:])


@pytest.mark.parametrize("V", [4096, 40000])
@pytest.mark.parametrize("once", [False, True])
def test_alpha_special_rows(V, once):
    """Identical rows give 1, disjoint one-hot rows give 0, masked (-inf) entries count as zero
    probability (at V = 40000 a whole chunk of row 2 is masked), and a constant added to a row changes
    nothing."""
    say(f"acceptance_rate special rows V={V} single-read={once}")
    r = torch.Generator(device=DEV).manual_seed(62)
    base = torch.randn((4, V), generator=r, device=DEV) * 3
    lp = base.clone()
    lq = base.clone()
    lp[1].fill_(-1e4)
    lp[1, 7] = 0.0
    lq[1].fill_(-1e4)
    lq[1, 4000] = 0.0
    lp[2, :V // 2] = -float("inf")
    lq[3] = lp[3] + 11.25
    with _handle() as h:
        a = _alpha(h, lp, lq, once=once)
    ref = oracle.acceptance_rate(to_np(lp), to_np(lq))
    assert abs(a[0] - 1.0) <= 1e-5
    assert a[1] <= 1e-6
    assert abs(a[2] - ref[2]) <= ALPHA_ABS
    assert abs(a[3] - 1.0) <= 1e-5


@pytest.mark.parametrize("bin_size,n_bins", [(2048, 21), (65536, 2)])
def test_bin_stats_on_given_values(bin_size, n_bins):
    """On the same fp32 values both sides take the same order statistics: the GPU's statistics are
    the oracle's rounded to fp32 (the mean within its float32 rounding).  Includes empty bins, a
    single-value bin, ties, negative positions and positions past the last bin; with 65536-position
    bins the first bin holds ~37000 values, more than the kernel stages on chip (its other path)."""
    say(f"acceptance_bin_stats on given values, bin_size={bin_size}")
    rng = np.random.default_rng(63)
    T = 40000
    alpha = (1 - rng.beta(0.3, 3, size=T)).astype(np.float32)
    alpha[::17] = 1.0                       # ties
    pos = rng.integers(0, 20 * 2048, size=T).astype(np.int32)
    pos[(pos >= 4 * 2048) & (pos < 5 * 2048)] = 3 * 2048        # bin 4 empty
    pos[(pos >= 7 * 2048) & (pos < 8 * 2048)] = -5               # bin 7 empty, those tokens ignored
    pos[10] = 7 * 2048 + 3                                        # bin 7: one value
    pos[11] = 25 * 2048                                           # beyond the bins (of 2048)
    with _handle() as h:
        for pc in (5.0, 0.0, 50.0, 100.0, 37.5):
            count = torch.empty(n_bins, dtype=torch.int32, device=DEV)
            mean = torch.empty(n_bins, dtype=torch.float32, device=DEV)
            pct = torch.empty(n_bins, dtype=torch.float32, device=DEV)
            sa.acceptance_bin_stats(h, torch.from_numpy(alpha).to(DEV), torch.from_numpy(pos).to(DEV), bin_size,
                                    n_bins, pc, count, mean, pct)
            assert sa.sparse_attn_check(h) == 0
            rc, rm, rp = oracle.bin_percentiles(alpha, pos, bin_size, n_bins, pc)
            np.testing.assert_array_equal(to_np(count), rc)
            gm, gp = to_np(mean), to_np(pct)
            for j in range(n_bins):
                if rc[j] == 0:
                    assert np.isnan(gm[j]) and np.isnan(gp[j]), j
                    continue
                # the same double arithmetic, up to a contraction into one fma: at most 1 ulp of fp32
                assert abs(gp[j] - np.float32(rp[j])) <= np.spacing(np.float32(rp[j])), (pc, j, gp[j], rp[j])
                assert abs(gm[j] - rm[j]) <= 1e-7 * max(1.0, abs(rm[j])), (j, gm[j], rm[j])


def test_pipeline_at_bench_size():
    """The measurement as the benchmark runs it: 4096 tokens over a 151936-entry vocabulary on the
    single-read path, the 5-percentile per bin of 2048 positions; alpha checked on sampled tokens, the statistics of the
    GPU's alphas against the oracle's statistics of its own alphas."""
    T, V = 4096, 151936
    say(f"acceptance pipeline T={T} V={V}")
    d = inputs.acceptance_inputs(T, V, DEV)
    with _handle() as h:
        alpha = torch.empty(T, dtype=torch.float32, device=DEV)
        sa.acceptance_rate(h, d["logits_p"], d["logits_q"], alpha, ws=sa.workspace(h, sa.SA_OP_ACCEPT, T, V))
        count = torch.empty(2, dtype=torch.int32, device=DEV)
        mean = torch.empty(2, dtype=torch.float32, device=DEV)
        pct = torch.empty(2, dtype=torch.float32, device=DEV)
        sa.acceptance_bin_stats(h, alpha, d["pos"], 2048, 2, 5.0, count, mean, pct)
        assert sa.sparse_attn_check(h) == 0
    rows = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(64).integers(0, T, 29)]))
    rt = torch.as_tensor(rows, device=DEV)
    ref_rows = oracle.acceptance_rate(to_np(d["logits_p"][rt]), to_np(d["logits_q"][rt]))
    ga = to_np(alpha)
    assert np.abs(ga[rows] - ref_rows).max() <= ALPHA_ABS
    # the statistics of all T tokens: the oracle's alphas, 256 rows at a time
    ref = np.concatenate([oracle.acceptance_rate(to_np(d["logits_p"][i:i + 256]), to_np(d["logits_q"][i:i + 256]))
                          for i in range(0, T, 256)])
    assert np.abs(ga - ref).max() <= ALPHA_ABS
    rc, rm, rp = oracle.bin_percentiles(ref, np.arange(T), 2048, 2, 5.0)
    np.testing.assert_array_equal(to_np(count), rc)
    assert np.abs(to_np(pct) - rp).max() <= ALPHA_ABS
    assert np.abs(to_np(mean) - rm).max() <= ALPHA_ABS
    say(f"  alpha mean {ref.mean():.4f}, 5-percentile per bin {rp}, max|d alpha|={np.abs(ga - ref).max():.2e}")
