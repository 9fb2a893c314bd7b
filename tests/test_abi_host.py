"""CPU checks of the C ABI: the library loads, exports every symbol the header declares,
and rejects bad configurations before touching a device."""
import ctypes
import os
import re

import pytest

import indexer_selected_sparse_scores_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("sparse_attn_create", "indexer_scores", "topk_select", "sparse_attn_prefill",
              "sparse_attn_decode"):
        assert n in names
    assert set(names) == set(sa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = sa.load_library()
    for n in _declared_functions():
        assert hasattr(lib, n), n


def _create(**over):
    lib = sa.load_library()
    c = sa.Config(**over).to_c()
    h = ctypes.c_void_p()
    st = lib.sparse_attn_create(ctypes.byref(c), ctypes.byref(h))
    return st, lib.sparse_attn_last_error(None).decode(), h


@pytest.mark.parametrize("over,needle", [
    (dict(max_topk=0), "max_topk"),
    (dict(max_topk=8193), "max_topk"),
    (dict(n_heads=16, n_kv_heads=3), "multiple"),
    (dict(d_v=600), "d_v"),
    (dict(page_size=0), "page_size"),
    (dict(softmax_scale=-1.0), "softmax_scale"),
    (dict(n_idx_heads=0), ">= 1"),
])
def test_create_rejects_bad_config(over, needle):
    st, msg, h = _create(**over)
    assert st == sa.SA_ERR_INVALID_ARG
    assert needle in msg
    assert not h.value


def test_create_null_arguments():
    lib = sa.load_library()
    h = ctypes.c_void_p()
    assert lib.sparse_attn_create(None, ctypes.byref(h)) == sa.SA_ERR_INVALID_ARG
    # calls with a NULL handle fail cleanly and touch no device
    assert lib.indexer_scores(None, None, None, None, 1, None, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill(None, *([None] * 6), 1, 1, None, None, None, None, 0, None) \
        == sa.SA_ERR_INVALID_ARG
    assert lib.topk_select_blocks(None, None, 1, 1, 1, None, None, 1, 64, 1, None, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill_blocks(None, *([None] * 6), 1, 1, 64, 1, None, None, None, None, 0, None) \
        == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_decode_blocks(None, *([None] * 6), 1, None, 1, None, None, 1, 1, 64, 1, None, None,
                                         None, None, 0, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill_paged(None, *([None] * 6), 1, None, 1, 1, None, None, 1, 1, 1, None, None, None,
                                         None, 0, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill_chunk(None, *([None] * 6), 1, None, 1, 0, 1, 1, None, None, None, None, 0,
                                         None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill_varlen(None, *([None] * 6), 1, None, 1, 1, None, None, 1, 1, 1, None, None, None,
                                          None, 0, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_decode_noalloc(None, *([None] * 6), 1, None, 1, None, None, 1, 1, None, None, None,
                                          None) == sa.SA_ERR_INVALID_ARG
    size = ctypes.c_size_t()
    assert lib.sparse_attn_workspace_size(None, 1, 1, 1, ctypes.byref(size)) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_last_error(None)
