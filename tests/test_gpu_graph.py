"""HIP graph capture of the library's calls: they allocate nothing and clear their counters and
histograms with kernels (no memset nodes), so a captured step replays to the eager result, bit for bit,
on every replay -- checked with eager work and synchronisations between the replays."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import indexer_selected_sparse_scores_amd as sa
from indexer_selected_sparse_scores_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _replays_match(run, outputs, n=3):
    """Eager reference, then capture `run` on a side stream and replay it n times, checking every replay."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # a warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        run()
    for i in range(n):
        for t in outputs:
            t.fill_(-7)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs, ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager result"
    say(f"  {n} replays equal to the eager result")


def test_decode_step_replays_from_a_graph():
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [5000, 129, 20000, 64, 777, 4097, 3, 16384]
    say(f"graph capture: sparse_attn_decode, ctx={ctx}")
    d = inputs.decode_inputs(inputs.small(wl, topk=2048), DEV, ctx=ctx, seed=41)
    with sa.Handle(inputs.library_config(wl)) as h:
        B = len(ctx)
        out = torch.empty((B, 16, 512), device=DEV)
        lse = torch.empty((B, 16), device=DEV)
        idx = torch.empty((B, 2048), device=DEV, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_DECODE, B, d["max_ctx"])

        def run():
            sa.sparse_attn_decode(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], None, d["kidx_pages"],
                                  d["block_table"], d["ctx_len"], d["topk"], d["max_ctx"], out, lse, idx, ws)

        _replays_match(run, [out, lse, idx])
        assert sa.sparse_attn_check(h) == 0


def test_prefill_replays_from_a_graph():
    wl = inputs.WORKLOADS["prefill_8k"]
    L = 2051
    say(f"graph capture: sparse_attn_prefill, L={L}, topk=256")
    P = inputs.prefill_inputs(wl, DEV, L=L, seed=42)
    with sa.Handle(inputs.library_config(wl, max_topk=256)) as h:
        out = torch.empty((L, 16, 512), device=DEV)
        lse = torch.empty((L, 16), device=DEV)
        idx = torch.empty((L, 256), device=DEV, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_PREFILL, L)

        def run():
            sa.sparse_attn_prefill(h, P["q"], P["k"], None, P["q_idx"], P["w"], P["k_idx"], 256, out, lse, idx, ws)

        _replays_match(run, [out, lse, idx])
        assert sa.sparse_attn_check(h) == 0


def test_two_tier_decode_replays_from_a_graph():
    wl = inputs.WORKLOADS["decode_b64"]
    ctx = [9000, 300, 20000, 4097]
    say(f"graph capture: sparse_attn_decode_blocks, ctx={ctx}")
    d = inputs.decode_inputs(inputs.small(wl, topk=2048), DEV, ctx=ctx, seed=43)
    with sa.Handle(inputs.library_config(wl)) as h:
        B = len(ctx)
        out = torch.empty((B, 16, 512), device=DEV)
        idx = torch.empty((B, 2048), device=DEV, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_DECODE_BLOCKS, B, d["max_ctx"])

        def run():
            sa.sparse_attn_decode_blocks(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], None, d["kidx_pages"],
                                         d["block_table"], d["ctx_len"], d["topk"], d["max_ctx"], 64, 48, out, None,
                                         idx, ws)

        _replays_match(run, [out, idx])
        assert sa.sparse_attn_check(h) == 0


def test_varlen_prefill_replays_from_a_graph():
    """The varlen prefill builds its tile table and row layout on the device, so the captured call replays
    to the eager result."""
    wl = inputs.small(inputs.WORKLOADS["decode_b64"], topk=512)
    ctx, n_new = [3000, 700, 64, 1500], [300, 700, 13, 9]
    say(f"graph capture: sparse_attn_prefill_varlen, ctx={ctx} new={n_new}")
    rs = np.concatenate([np.full(k, b) for b, k in enumerate(n_new)])
    rp = np.concatenate([np.arange(c - k, c) for c, k in zip(ctx, n_new)])
    d = inputs.paged_rows_inputs(wl, ctx, rs, rp, DEV, seed=43)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).to(DEV)
    ctx_len = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).to(DEV)
    T = len(rs)
    with sa.Handle(inputs.library_config(wl, max_topk=512)) as h:
        s = h.cfg
        out = torch.empty((T, s.n_heads, s.d_v), device=DEV)
        lse = torch.empty((T, s.n_heads), device=DEV)
        idx = torch.empty((T, 512), device=DEV, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_PREFILL_VARLEN, T, max(ctx))

        def run():
            sa.sparse_attn_prefill_varlen(h, d["q"], d["q_idx"], d["w"], d["kv_pages"], d["v_pages"],
                                          d["kidx_pages"], d["block_table"], cu, ctx_len, max(ctx), 512, out, lse,
                                          idx, ws)

        _replays_match(run, [out, lse, idx])
        assert sa.sparse_attn_check(h) == 0


def test_query_projection_replays_from_a_graph():
    """The query projection is one kernel with no workspace and no library handle, so it captures."""
    L, K = 777, 16 * 576
    say(f"graph capture: indexer_project_q, L={L}")
    g = torch.Generator(device=DEV).manual_seed(44)
    q = torch.randn((L, K), generator=g, device=DEV).to(torch.bfloat16)
    W_iq = (torch.randn((8192, K), generator=g, device=DEV) * K ** -0.5).to(torch.bfloat16)
    W_w = (torch.randn((64, K), generator=g, device=DEV) * K ** -0.5).to(torch.bfloat16)
    with sa.Handle(inputs.library_config(inputs.WORKLOADS["decode_b64"])) as h:
        q_idx = torch.empty((L, 8192), device=DEV, dtype=torch.bfloat16)
        w = torch.empty((L, 64), device=DEV)

        def run():
            sa.indexer_project_q(h, q, W_iq, W_w, q_idx, w)

        _replays_match(run, [q_idx, w])
        assert sa.sparse_attn_check(h) == 0


def test_acceptance_rate_replays_from_a_graph():
    """The single-read acceptance rate refills its exchange words with a kernel before every run, so a
    captured call (with the per-bin statistics) replays to the eager result; the two-pass call as well."""
    T, V = 300, 151936
    say(f"graph capture: acceptance_rate T={T} V={V}, both paths, and acceptance_bin_stats")
    d = inputs.acceptance_inputs(T, V, DEV, seed=66)
    with sa.Handle(sa.Config()) as h:
        ws = sa.workspace(h, sa.SA_OP_ACCEPT, T, V)
        a1 = torch.empty(T, dtype=torch.float32, device=DEV)
        a2 = torch.empty(T, dtype=torch.float32, device=DEV)
        count = torch.empty(1, dtype=torch.int32, device=DEV)
        mean = torch.empty(1, dtype=torch.float32, device=DEV)
        pct = torch.empty(1, dtype=torch.float32, device=DEV)

        def run():  # on the current stream: the capture stream while capturing
            sa.acceptance_rate(h, d["logits_p"], d["logits_q"], a1, ws=ws)
            sa.acceptance_rate(h, d["logits_p"], d["logits_q"], a2)
            sa.acceptance_bin_stats(h, a1, d["pos"], 2048, 1, 5.0, count, mean, pct)

        _replays_match(run, [a1, a2, count, mean, pct])
        assert sa.sparse_attn_check(h) == 0
        assert (a1 - a2).abs().max().item() <= 1e-4
