"""CPU tests of the library's host-side argument checks, through the C ABI on a host-only handle
(sparse_attn_create_host): it touches no device, so every call stops either at its validation (with the
status a bad argument must give) or, with valid arguments, right after it with SA_ERR_UNSUPPORTED and
"launches nothing".  Pointers are fake device addresses: the checks never dereference them."""
import ctypes

import pytest

import indexer_selected_sparse_scores_amd as sa

A = 0x7F0000000000       # a 16-byte aligned fake device address
M = A + 4                # a misaligned one
PASSED = sa.SA_ERR_UNSUPPORTED  # validation passed; a host-only handle launches nothing


def status(h, fn, *args):
    return getattr(sa.load_library(), fn)(h.ptr, *args)


def passed(h, fn, *args):
    st = status(h, fn, *args)
    return st == PASSED and "launches nothing" in sa.sparse_attn_last_error(h)


@pytest.fixture(scope="module")
def h():
    with sa.Handle(sa.Config(max_topk=2048), host_cus=256) as hh:
        yield hh


def ws_size(h, op, n, max_ctx=0):
    return sa.sparse_attn_workspace_size(h, op, n, max_ctx)


def test_host_handle_config_checks():
    lib = sa.load_library()
    c = sa.Config(max_topk=0).to_c()
    out = ctypes.c_void_p()
    assert lib.sparse_attn_create_host(ctypes.byref(c), 256, ctypes.byref(out)) == sa.SA_ERR_INVALID_ARG
    assert "max_topk" in lib.sparse_attn_last_error(None).decode() and not out.value
    c = sa.Config().to_c()
    assert lib.sparse_attn_create_host(ctypes.byref(c), 0, ctypes.byref(out)) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_create_host(ctypes.byref(c), 256, ctypes.byref(out)) == sa.SA_OK
    lib.sparse_attn_destroy(out)


def test_host_handle_sizes_and_launches_nothing(h):
    assert ws_size(h, sa.SA_OP_DECODE, 64, 131072) > 64 * 131072 * 4  # the decode scores alone
    assert ws_size(h, sa.SA_OP_PREFILL, 131072) > 131072 * 2048 * 4    # the index lists alone
    assert status(h, "sparse_attn_check", None, None) == PASSED


def prefill_args(h, L=1000, topk=64, ws=None, **over):
    a = dict(q=A, k=A, v=None, q_idx=A, w=A, k_idx=A, L=L, topk=topk, out=A, lse=None, idx=None,
             ws=A, ws_bytes=ws if ws is not None else ws_size(h, sa.SA_OP_PREFILL, L), stream=None)
    a.update(over)
    return list(a.values())


def test_prefill_checks(h):
    assert passed(h, "sparse_attn_prefill", *prefill_args(h))
    for name in ("q", "k", "q_idx", "w", "k_idx", "out"):
        assert status(h, "sparse_attn_prefill", *prefill_args(h, **{name: M})) == sa.SA_ERR_INVALID_ARG, name
        assert "aligned" in sa.sparse_attn_last_error(h)
        assert status(h, "sparse_attn_prefill", *prefill_args(h, **{name: None})) == sa.SA_ERR_INVALID_ARG, name
    assert status(h, "sparse_attn_prefill", *prefill_args(h, v=A)) == sa.SA_ERR_INVALID_ARG  # v with v_from_k
    assert status(h, "sparse_attn_prefill", *prefill_args(h, topk=2049)) == sa.SA_ERR_INVALID_ARG
    assert "max_topk" in sa.sparse_attn_last_error(h)
    assert status(h, "sparse_attn_prefill", *prefill_args(h, topk=0)) == sa.SA_ERR_INVALID_ARG
    assert status(h, "sparse_attn_prefill", *prefill_args(h, L=0, ws=0)) == sa.SA_ERR_INVALID_ARG
    need = ws_size(h, sa.SA_OP_PREFILL, 1000)
    assert status(h, "sparse_attn_prefill", *prefill_args(h, ws=need - 1)) == sa.SA_ERR_WORKSPACE
    args = prefill_args(h)
    args[11] = None  # no workspace pointer
    assert status(h, "sparse_attn_prefill", *args) == sa.SA_ERR_WORKSPACE


def decode_args(h, B=64, max_ctx=131072, ws=None, **over):
    a = dict(q=A, q_idx=A, w=A, kv=A, v=None, kidx=A, n_pages=131072, table=A, max_blocks=2048, ctx=A, topk=A,
             B=B, max_ctx=max_ctx, out=A, lse=None, idx=None, ws=A,
             ws_bytes=ws if ws is not None else ws_size(h, sa.SA_OP_DECODE, B, max_ctx), stream=None)
    a.update(over)
    return list(a.values())


def test_decode_checks(h):
    assert passed(h, "sparse_attn_decode", *decode_args(h))
    for name in ("q", "q_idx", "w", "kv", "kidx", "out"):
        assert status(h, "sparse_attn_decode", *decode_args(h, **{name: M})) == sa.SA_ERR_INVALID_ARG, name
        assert status(h, "sparse_attn_decode", *decode_args(h, **{name: None})) == sa.SA_ERR_INVALID_ARG, name
    for name in ("table", "ctx", "topk"):
        assert status(h, "sparse_attn_decode", *decode_args(h, **{name: None})) == sa.SA_ERR_INVALID_ARG, name
    assert status(h, "sparse_attn_decode", *decode_args(h, max_ctx=2048 * 64 + 1, ws=1 << 40)) == sa.SA_ERR_INVALID_ARG
    assert status(h, "sparse_attn_decode", *decode_args(h, B=0, ws=0)) == sa.SA_ERR_INVALID_ARG
    assert status(h, "sparse_attn_decode", *decode_args(h, B=65536, ws=0)) == sa.SA_ERR_INVALID_ARG
    assert status(h, "sparse_attn_decode", *decode_args(h, n_pages=0)) == sa.SA_ERR_INVALID_ARG
    need = ws_size(h, sa.SA_OP_DECODE, 64, 131072)
    assert status(h, "sparse_attn_decode", *decode_args(h, ws=need - 1)) == sa.SA_ERR_WORKSPACE
    # the two-tier decode: block-size rule on top of the same checks
    blk = decode_args(h)
    assert status(h, "sparse_attn_decode_blocks", *(blk[:13] + [48, 64] + blk[13:])) == sa.SA_ERR_INVALID_ARG
    assert status(h, "sparse_attn_decode_blocks", *(blk[:13] + [64, 512] + blk[13:])) == sa.SA_ERR_UNSUPPORTED
    assert "16384" in sa.sparse_attn_last_error(h)
    assert passed(h, "sparse_attn_decode_blocks", *(blk[:13] + [64, 64] + blk[13:]))


def test_decode_noalloc_checks(h):
    args = decode_args(h)
    no_ws = args[:17] + [None]
    assert passed(h, "sparse_attn_decode_noalloc", *no_ws)
    big = decode_args(h, max_ctx=1 << 20, max_blocks=1 << 14)[:17] + [None]
    assert status(h, "sparse_attn_decode_noalloc", *big) == sa.SA_ERR_UNSUPPORTED
    assert "allocation-free" in sa.sparse_attn_last_error(h)


def test_paged_rows_chunk_varlen_checks(h):
    T, max_ctx = 300, 5000
    ws = ws_size(h, sa.SA_OP_PREFILL_PAGED, T, max_ctx)
    good = [A, A, A, A, None, A, 100, A, 2, 100, A, A, T, max_ctx, 64, A, None, None, A, ws, None]
    assert passed(h, "sparse_attn_prefill_paged", *good)
    bad = list(good); bad[0] = M
    assert status(h, "sparse_attn_prefill_paged", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[10] = None  # row_seq
    assert status(h, "sparse_attn_prefill_paged", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[13] = 100 * 64 + 1  # max_ctx beyond the block table
    assert status(h, "sparse_attn_prefill_paged", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[14] = 4096  # topk > max_topk
    assert status(h, "sparse_attn_prefill_paged", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[19] = ws - 1
    assert status(h, "sparse_attn_prefill_paged", *bad) == sa.SA_ERR_WORKSPACE

    C, pos0 = 512, 4000
    ws = ws_size(h, sa.SA_OP_PREFILL_CHUNK, C, pos0 + C)
    good = [A, A, A, A, None, A, 100, A, 100, pos0, C, 64, A, None, None, A, ws, None]
    assert passed(h, "sparse_attn_prefill_chunk", *good)
    bad = list(good); bad[5] = M  # kidx_pages
    assert status(h, "sparse_attn_prefill_chunk", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[9] = 100 * 64 - C + 1  # pos0 + C beyond the block-table row
    assert status(h, "sparse_attn_prefill_chunk", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[10] = 0
    assert status(h, "sparse_attn_prefill_chunk", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[16] = ws - 1
    assert status(h, "sparse_attn_prefill_chunk", *bad) == sa.SA_ERR_WORKSPACE

    ws = ws_size(h, sa.SA_OP_PREFILL_VARLEN, T, max_ctx)
    good = [A, A, A, A, None, A, 100, A, 4, 100, A, A, T, max_ctx, 64, A, None, None, A, ws, None]
    assert passed(h, "sparse_attn_prefill_varlen", *good)
    bad = list(good); bad[2] = M  # w
    assert status(h, "sparse_attn_prefill_varlen", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[10] = None  # cu_seqlens
    assert status(h, "sparse_attn_prefill_varlen", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[8] = 0  # n_seqs
    assert status(h, "sparse_attn_prefill_varlen", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[14] = 0
    assert status(h, "sparse_attn_prefill_varlen", *bad) == sa.SA_ERR_INVALID_ARG
    bad = list(good); bad[19] = ws - 1
    assert status(h, "sparse_attn_prefill_varlen", *bad) == sa.SA_ERR_WORKSPACE


def test_indexer_topk_checks(h):
    assert passed(h, "indexer_scores", A, A, A, 1000, A, None)
    assert status(h, "indexer_scores", M, A, A, 1000, A, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "indexer_scores", A, A, A, 0, A, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "indexer_scores", A, A, A, 16385, A, None) == sa.SA_ERR_UNSUPPORTED
    assert "16384" in sa.sparse_attn_last_error(h)
    assert passed(h, "topk_select", A, 10, 100, 100, None, None, 64, A, None)
    assert status(h, "topk_select", A, 10, 100, 99, None, None, 64, A, None) == sa.SA_ERR_INVALID_ARG  # ld < cols
    assert status(h, "topk_select", A, 10, 100, 100, None, None, 2049, A, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "topk_select", A, 0, 100, 100, None, None, 64, A, None) == sa.SA_ERR_INVALID_ARG
    assert passed(h, "topk_select_blocks", A, 10, 1000, 1000, None, None, 64, 64, 16, A, None)
    assert status(h, "topk_select_blocks", A, 10, 1000, 1000, None, None, 64, 63, 16, A, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "topk_select_blocks", A, 10, 1000, 1000, None, None, 64, 64, 0, A, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "topk_select_blocks", A, 10, 1000, 1000, None, None, 64, 1024, 17, A, None) == sa.SA_ERR_UNSUPPORTED


def test_projection_acceptance_checks(h):
    assert ws_size(h, sa.SA_OP_PROJECT, 100) == 0  # the query projection needs no workspace
    assert passed(h, "indexer_project_q", A, 100, A, A, A, A, None, 0, None)
    assert status(h, "indexer_project_q", M, 100, A, A, A, A, None, 0, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "indexer_project_q", A, 100, A, None, A, A, None, 0, None) == sa.SA_ERR_INVALID_ARG  # half a pair
    assert status(h, "indexer_project_q", A, 100, None, None, None, None, None, 0, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "indexer_project_q", A, 0, A, A, A, A, None, 0, None) == sa.SA_ERR_INVALID_ARG
    with sa.Handle(sa.Config(d_idx=96), host_cus=256) as odd:  # H_I * d_I = 6144: a multiple of 256
        assert passed(odd, "indexer_project_q", A, 100, A, A, A, A, None, 0, None)
    with sa.Handle(sa.Config(n_idx_heads=3, d_idx=64), host_cus=256) as odd:  # H_I * d_I = 192
        assert status(odd, "indexer_project_q", A, 100, A, A, A, A, None, 0, None) == sa.SA_ERR_UNSUPPORTED
        assert "multiple of 256" in sa.sparse_attn_last_error(odd)
    assert passed(h, "indexer_project_k", A, 100, A, A, None, 0, 0, 0, None, None, 0, None)
    assert status(h, "indexer_project_k", A, 100, M, A, None, 0, 0, 0, None, None, 0, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "indexer_project_k", A, 100, A, A, A, 0, 10, 10, None, None, 0, None) == sa.SA_ERR_INVALID_ARG
    assert passed(h, "acceptance_rate", A, A, 100, 1000, 1000, A, None, 0, None)
    assert status(h, "acceptance_rate", A, A, 100, 1000, 999, A, None, 0, None) == sa.SA_ERR_INVALID_ARG
    # the single-read path: per token and chunk of 3520 float4 per row, 2 state words and 11 partials
    need = ws_size(h, sa.SA_OP_ACCEPT, 100, 151936)
    assert need == 100 * 11 * (16 + 11 * 4)
    assert passed(h, "acceptance_rate", A, A, 100, 151936, 151936, A, A, need, None)
    assert status(h, "acceptance_rate", A, A, 100, 151936, 151936, A, A, need - 1, None) == sa.SA_ERR_WORKSPACE
    assert ws_size(h, sa.SA_OP_ACCEPT, 100, 1001) == 0          # V % 4 != 0: two passes only
    assert ws_size(h, sa.SA_OP_ACCEPT, 100, 4 * 3520 * 33) == 0  # more than 32 workgroups per token
    assert ws_size(h, sa.SA_OP_ACCEPT, 1, 4) == 1 * 1 * (16 + 11 * 4)
    assert passed(h, "acceptance_rate", A, A, 100, 1001, 1001, A, A, 1, None)  # a workspace it does not need
    with sa.Handle(sa.Config(), host_cus=4) as few:              # 11 workgroups per token on 4 CUs
        assert ws_size(few, sa.SA_OP_ACCEPT, 100, 151936) == 0
    assert passed(h, "acceptance_bin_stats", A, A, 100, 2048, 1, ctypes.c_float(5.0), A, A, A, None)
    assert status(h, "acceptance_bin_stats", A, A, 100, 2048, 1, ctypes.c_float(100.5), A, A, A, None) \
        == sa.SA_ERR_INVALID_ARG
    assert status(h, "acceptance_bin_stats", A, A, 100, 0, 1, ctypes.c_float(5.0), A, A, A, None) \
        == sa.SA_ERR_INVALID_ARG


def test_measurement_aids_launch_nothing(h):
    assert status(h, "sparse_attn_peak_mfma", A, 10, A, A, None) == sa.SA_ERR_UNSUPPORTED
    assert status(h, "sparse_attn_peak_mfma", M, 10, A, A, None) == sa.SA_ERR_INVALID_ARG
    assert status(h, "sparse_attn_peak_stream", A, None, 1 << 20, A, None) == sa.SA_ERR_UNSUPPORTED
    assert status(h, "sparse_attn_peak_stream", A, None, 17, A, None) == sa.SA_ERR_INVALID_ARG
