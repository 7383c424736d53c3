"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects host-checkable bad arguments before touching the (absent) GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_topk.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    """Every function any include/*.h declares (comments stripped)."""
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:topk|indexer|hisparse)_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def T():
    from sparse_attention_indexer_amd import topk
    topk.load_library()
    return topk


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("topk_query_sizes", "topk_plan", "topk_select_paged", "topk_workspace_init",
              "topk_read_status", "topk_status_string", "topk_register_capacity", "topk_debug_keys",
              "topk_debug_stream_read", "topk_stream_read_groups",
              "topk_select_paged_timed", "topk_debug_histogram", "indexer_key_prologue", "indexer_debug_fp8", "indexer_query_prologue", "indexer_mqa_logits",
              "hisparse_resolve"):
        assert n in names


def test_every_declared_symbol_is_exported(T):
    lib = T.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(T):
    lib = T.load_library()
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.topk_status_string(st)
    assert lib.topk_status_string(-99) == b"unknown status"


def test_register_capacity(T):
    assert T.topk_register_capacity() == 32768


@pytest.mark.parametrize("kw", [
    dict(k=0), dict(k=2049), dict(max_rows=0), dict(max_len=-1), dict(max_len=1 << 31),
    dict(force_path=4), dict(force_path=-1), dict(wg_per_row=1), dict(wg_per_row=-2),
    dict(cand_capacity=-1), dict(min_chunk=-5), dict(spin_limit=-2),
])
def test_bad_config_rejected_without_gpu(T, kw):
    base = dict(k=2048, max_rows=7, max_len=80_000)
    base.update(kw)
    cfg = T.make_config(**base)
    with pytest.raises(T.TopKError) as e:
        T.topk_query_sizes(cfg)
    assert e.value.status == T.TOPK_ERR_INVALID_ARG


def test_reserved_must_be_zero(T):
    cfg = T.make_config(2048, 7, 80_000)
    cfg.reserved[2] = 1
    with pytest.raises(T.TopKError) as e:
        T.topk_query_sizes(cfg)
    assert e.value.status == T.TOPK_ERR_INVALID_ARG


def test_register_path_too_long_is_unsupported(T):
    cfg = T.make_config(2048, 2, 32769, force_path="register")
    with pytest.raises(T.TopKError) as e:
        T.topk_query_sizes(cfg)
    assert e.value.status == T.TOPK_ERR_UNSUPPORTED


def test_null_arguments_rejected(T):
    lib = T.load_library()
    cfg = T.make_config(2048, 7, 80_000)
    assert lib.topk_query_sizes(ctypes.byref(cfg), None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_query_sizes(None, None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_workspace_init(None, 256, None) == T.TOPK_ERR_INVALID_ARG
    v = ctypes.c_int32(0)
    assert lib.topk_read_status(None, 256, ctypes.byref(v), None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_debug_keys(None, 5, None, None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_debug_stream_read(None, 8, None, None, None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_debug_stream_read(None, -1, None, None, None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_stream_read_groups() >= 1
    assert lib.topk_debug_histogram(None, 0, None, 3, 2048, None, None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_debug_histogram(None, 0, None, 0, 0, None, None, None) == T.TOPK_ERR_INVALID_ARG
    bad = T.make_config(0, 7, 80_000)
    assert lib.topk_plan(ctypes.byref(bad), None, 7, None, 0, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_select_paged(ctypes.byref(bad), None, None, 0, None, 7, None, 0, 64,
                                 None, None, 2048, None, 0, None) == T.TOPK_ERR_INVALID_ARG
    good = T.make_config(2048, 7, 80_000)
    assert lib.topk_select_paged_timed(ctypes.byref(good), None, None, 0, None, 7, None, 0, 64,
                                       None, None, 2048, None, 0, None, None, None) == T.TOPK_ERR_INVALID_ARG


def test_valid_config_needs_a_device(T):
    """With no GPU in this container a valid configuration reaches the device
    query and reports a HIP error rather than crashing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(T.TopKError) as e:
        T.topk_query_sizes(T.make_config(2048, 7, 80_000))
    assert e.value.status == T.TOPK_ERR_HIP


def test_binding_rejects_strided_lengths_and_tables(T):
    """A strided view of the lengths or a block table without unit page
    stride would be read as other data by the library: the binding refuses
    both before any device call."""
    import torch
    lengths = torch.arange(14, dtype=torch.int32)[::2]
    table = torch.zeros((4, 8), dtype=torch.int32).t()
    ok_table = torch.zeros((4, 8), dtype=torch.int32)
    cfg = T.make_config(2048, 7, 80_000)
    with pytest.raises(ValueError, match="lengths"):
        T.topk_plan(cfg, lengths, torch.zeros(16, dtype=torch.int32))
    with pytest.raises(ValueError, match="lengths"):
        T._select_args(cfg, None, None, lengths, ok_table, 0, 64, None, None, None, None)
    with pytest.raises(ValueError, match="block_table"):
        T._select_args(cfg, None, None, lengths.contiguous(), table, 8, 64, None, None, None, None)


# --- the key prologue's host checks --------------------------------------------

def _key_cfg(**kw):
    from sparse_attention_indexer_amd import prologue as K
    base = dict(dim=128, rope_dim=64, eps=1e-6, page_size=64, max_pos=1000)
    base.update(kw)
    return K.indexer_key_config(base["dim"], base["rope_dim"], base["eps"], base["page_size"], base["max_pos"],
                                (ctypes.c_int32 * 3)())


@pytest.mark.parametrize("kw", [dict(dim=64), dict(rope_dim=12), dict(rope_dim=136), dict(rope_dim=-8),
                                dict(page_size=0), dict(max_pos=0), dict(eps=-1.0), dict(eps=float("nan")),
                                dict(eps=float("inf"))])
def test_key_prologue_bad_config_rejected_without_gpu(T, kw):
    from sparse_attention_indexer_amd import prologue as K
    lib = K._lib()
    buf = (ctypes.c_uint8 * 4096)()
    p = ctypes.addressof(buf)
    p16 = p + (-p % 16)
    cfg = _key_cfg(**kw)
    st = lib.indexer_key_prologue(ctypes.byref(cfg), p16, 128, 4, p16, p16, p16, p16, None, p16, 0, p16, p16,
                                  8, None, None)
    assert st == T.TOPK_ERR_INVALID_ARG


def test_key_prologue_bad_arguments_rejected_without_gpu(T):
    from sparse_attention_indexer_amd import prologue as K
    lib = K._lib()
    buf = (ctypes.c_uint8 * 4096)()
    p = ctypes.addressof(buf)
    a = p + (-p % 16)
    cfg = _key_cfg()
    call = lambda *args: lib.indexer_key_prologue(ctypes.byref(cfg), *args)   # noqa: E731
    ok = [a, 128, 4, a, a, a, a, None, a, 0, a, a, 8, None, None]
    bad = [
        (1, 120), (1, 130), (2, -1), (0, None), (3, None), (5, None), (8, None), (10, None), (11, None),
        (12, 0), (9, -1), (0, a + 2), (10, a + 8),
    ]
    for i, v in bad:
        args = list(ok)
        args[i] = v
        assert call(*args) == T.TOPK_ERR_INVALID_ARG, (i, v)
    args = list(ok)
    args[2] = 0
    assert call(*args) == T.TOPK_OK                       # no tokens: nothing to do, nothing enqueued
    assert lib.indexer_debug_fp8(None, 5, None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.indexer_debug_fp8(None, 0, None, None) == T.TOPK_OK
