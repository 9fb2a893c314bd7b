"""GPU test of sparse_attn_decode_noalloc, the decode step that allocates nothing: through the C ABI its
outputs equal sparse_attn_decode's (same kernels, the library's device array in place of the caller's
workspace) on two calls in a row, the second smaller than the first; a step larger than the array is
rejected before any launch."""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_scores_amd as sa
from indexer_selected_sparse_scores_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[no_alloc] {msg}", flush=True)


def _run(h, d, noalloc):
    B = d["q"].shape[0]
    K = h.cfg.max_topk
    out = torch.full((B, 16, 512), float("nan"), device=DEV)
    lse = torch.full((B, 16), float("nan"), device=DEV)
    idx = torch.full((B, K), -7, device=DEV, dtype=torch.int32)
    args = (h, d["q"], d["q_idx"], d["w"], d["kv_pages"], None, d["kidx_pages"], d["block_table"], d["ctx_len"],
            d["topk"], d["max_ctx"], out, lse, idx)
    if noalloc:
        sa.sparse_attn_decode_noalloc(*args)
    else:
        ws = sa.workspace(h, sa.SA_OP_DECODE, B, d["max_ctx"])
        sa.sparse_attn_decode(*args, ws)
    assert sa.sparse_attn_check(h) == 0
    torch.cuda.synchronize()
    return out, lse, idx


def test_noalloc_decode_equals_workspace_decode():
    torch.cuda.set_device(0)
    wl = inputs.WORKLOADS["decode_b64"]
    cases = [
        # larger first: 8 sequences with contexts up to 40000, budget 2048
        (2048, [1, 63, 2049, 5000, 40000, 9000, 131, 17000], 21),
        # then smaller: the array keeps the first call's contents, which must not leak into this one
        (256, [300, 1, 77, 2600], 22),
    ]
    for K, ctx, seed in cases:
        say(f"decode B={len(ctx)} ctx={ctx} topk={K}, workspace call then allocation-free call")
        d = inputs.decode_inputs(inputs.small(wl, topk=K), DEV, ctx=ctx, seed=seed)
        with sa.Handle(inputs.library_config(wl, max_topk=K)) as h:
            ref = _run(h, d, noalloc=False)
            got = _run(h, d, noalloc=True)
        for name, r, g in zip(("out", "lse", "idx"), ref, got):
            assert torch.equal(r, g), f"{name} differs (ctx={ctx}, topk={K})"
        gi = got[2].cpu().numpy()
        for b, n in enumerate(ctx):
            m = min(K, n)
            assert np.all(gi[b][:m] >= 0) and np.all(gi[b][m:] == -1), f"seq {b}"


def test_noalloc_decode_rejects_oversized_step():
    torch.cuda.set_device(0)
    wl = inputs.WORKLOADS["decode_b64"]
    say("decode B=64 max_ctx=1048576: beyond the 64 MiB array, rejected on the host")
    with sa.Handle(inputs.library_config(wl)) as h:
        lib = sa.load_library()
        st = lib.sparse_attn_decode_noalloc(h.ptr, *([None] * 6), 1, None, 16384, None, None, 64, 1 << 20,
                                            None, None, None, None)
        assert st == sa.SA_ERR_UNSUPPORTED
        assert "allocation-free" in sa.sparse_attn_last_error(h)
