"""ctypes binding of the indexer key prologue (include/indexer_prologue.h), in
``libsparse_topk.so``.

Argument marshalling only: LayerNorm, rotary embedding, FP8 quantization and
the cache store all run in the library's HIP kernel. There is no fallback: if
the library is missing or a call fails, these functions raise.
"""
from __future__ import annotations

import ctypes

import torch

from . import topk

KEY_DIM = 128
DEVICE_BAD_POSITION = 0x100
DEVICE_BAD_SLOT = 0x200


class indexer_key_config(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("eps", ctypes.c_float),
                ("page_size", ctypes.c_int32), ("max_pos", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 3)]


_bound = False


def _lib():
    global _bound
    lib = topk.load_library()
    if not _bound:
        V, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.indexer_key_prologue.argtypes = [ctypes.POINTER(indexer_key_config), V, I64, I32, V, V, V, V, V, V,
                                             I64, V, V, I64, V, V]
        lib.indexer_key_prologue.restype = ctypes.c_int
        lib.indexer_debug_fp8.argtypes = [V, I64, V, V]
        lib.indexer_debug_fp8.restype = ctypes.c_int
        lib.indexer_query_prologue.argtypes = [V, I32, I32, V, ctypes.c_float, V, I32, I32, V, V, V, V, V]
        lib.indexer_query_prologue.restype = ctypes.c_int
        _bound = True
    return lib


def _need(t: torch.Tensor, dtypes, name: str) -> None:
    if t.dtype not in dtypes or not t.is_cuda:
        raise TypeError(f"{name} must be a {' or '.join(map(str, dtypes))} tensor on the GPU")


def indexer_key_prologue(k_act: torch.Tensor, ln_weight: torch.Tensor, ln_bias: torch.Tensor, eps: float,
                         cos_sin: torch.Tensor | None, rope_dim: int, positions: torch.Tensor,
                         token_row: torch.Tensor | None, block_table: torch.Tensor, bt_row_stride: int,
                         page_size: int, cache_fp8: torch.Tensor, cache_scale: torch.Tensor,
                         status: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue the fused key path for k_act.shape[0] tokens (see the header).

    k_act: bfloat16 or int16/uint16 bits [T, >=128] with unit inner stride;
    cos_sin: float32 [max_pos, rope_dim]; cache_fp8: uint8 [slots, 128];
    cache_scale: float32 [slots]; status: int32 [1] or None."""
    _need(k_act, (torch.bfloat16, torch.int16, torch.uint16), "k_act")
    if k_act.dim() != 2 or (k_act.numel() > 0 and k_act.stride(1) != 1):
        raise ValueError("k_act must be 2-D with unit stride along dims")
    k_stride = k_act.stride(0) if k_act.shape[0] > 0 else KEY_DIM   # (an empty tensor's stride is arbitrary)
    for t, name in ((ln_weight, "ln_weight"), (ln_bias, "ln_bias"), (cache_scale, "cache_scale")):
        _need(t, (torch.float32,), name)
    _need(positions, (torch.int32,), "positions")
    _need(block_table, (torch.int32,), "block_table")
    _need(cache_fp8, (torch.uint8,), "cache_fp8")
    if token_row is not None:
        _need(token_row, (torch.int32,), "token_row")
    if not all(t.is_contiguous() for t in (positions, ln_weight, ln_bias, cache_fp8, cache_scale)):
        raise ValueError("positions, LayerNorm parameters and the cache must be contiguous")
    if token_row is not None and not token_row.is_contiguous():
        raise ValueError("token_row must be contiguous")
    if block_table.dim() > 0 and block_table.stride(-1) != 1:
        raise ValueError("block_table must have unit stride along pages")
    max_pos = 1
    if rope_dim:
        if cos_sin is None:
            raise ValueError("rope_dim > 0 needs cos_sin")
        _need(cos_sin, (torch.float32,), "cos_sin")
        if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != rope_dim:
            raise ValueError("cos_sin must be a contiguous [max_pos, rope_dim] table")
        max_pos = cos_sin.shape[0]
    elif cos_sin is not None:
        max_pos = cos_sin.shape[0]
    else:
        max_pos = 2 ** 31 - 1
    if cache_fp8.dim() != 2 or cache_fp8.shape[1] != KEY_DIM or cache_scale.numel() != cache_fp8.shape[0]:
        raise ValueError("cache_fp8 must be [slots, 128] and cache_scale [slots]")
    cfg = indexer_key_config(KEY_DIM, int(rope_dim), float(eps), int(page_size), int(max_pos),
                             (ctypes.c_int32 * 3)())
    st = _lib().indexer_key_prologue(
        ctypes.byref(cfg), k_act.data_ptr(), k_stride, k_act.shape[0], ln_weight.data_ptr(),
        ln_bias.data_ptr(), None if cos_sin is None else cos_sin.data_ptr(), positions.data_ptr(),
        None if token_row is None else token_row.data_ptr(), block_table.data_ptr(), int(bt_row_stride),
        cache_fp8.data_ptr(), cache_scale.data_ptr(), cache_fp8.shape[0],
        None if status is None else status.data_ptr(), topk._stream(stream))
    topk._check("indexer_key_prologue", st)


def indexer_query_prologue(q_act: torch.Tensor, w_raw: torch.Tensor, gate_scale: float,
                           cos_sin: torch.Tensor | None, rope_dim: int, positions: torch.Tensor,
                           status: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Enqueue the fused query path; returns (q_codes uint8 [T, H, 128], w_out
    float32 [T, H]) allocated here by torch (the library itself allocates nothing).

    q_act: bfloat16 or int16/uint16 bits [T, H, 128], contiguous; w_raw float32 [T, H]."""
    _need(q_act, (torch.bfloat16, torch.int16, torch.uint16), "q_act")
    _need(w_raw, (torch.float32,), "w_raw")
    _need(positions, (torch.int32,), "positions")
    if q_act.dim() != 3 or q_act.shape[2] != KEY_DIM or not q_act.is_contiguous():
        raise ValueError("q_act must be a contiguous [tokens, heads, 128] tensor")
    T, H = q_act.shape[0], q_act.shape[1]
    if tuple(w_raw.shape) != (T, H) or not w_raw.is_contiguous() or positions.numel() != T:
        raise ValueError("w_raw must be [tokens, heads] and positions [tokens]")
    max_pos = 2 ** 31 - 1
    if rope_dim:
        if cos_sin is None:
            raise ValueError("rope_dim > 0 needs cos_sin")
        _need(cos_sin, (torch.float32,), "cos_sin")
        if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != rope_dim:
            raise ValueError("cos_sin must be a contiguous [max_pos, rope_dim] table")
        max_pos = cos_sin.shape[0]
    codes = torch.empty((T, H, KEY_DIM), dtype=torch.uint8, device=q_act.device)
    w_out = torch.empty((T, H), dtype=torch.float32, device=q_act.device)
    st = _lib().indexer_query_prologue(q_act.data_ptr(), T, H, w_raw.data_ptr(), float(gate_scale),
                                       None if cos_sin is None else cos_sin.data_ptr(), int(rope_dim), int(max_pos),
                                       positions.data_ptr(), codes.data_ptr(), w_out.data_ptr(),
                                       None if status is None else status.data_ptr(), topk._stream(stream))
    topk._check("indexer_query_prologue", st)
    return codes, w_out


def debug_fp8(x: torch.Tensor, stream=None) -> torch.Tensor:
    """The kernel's own FP32 -> E4M3 conversion of every element of x."""
    _need(x, (torch.float32,), "x")
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    st = _lib().indexer_debug_fp8(x.data_ptr(), x.numel(), out.data_ptr(), topk._stream(stream))
    topk._check("indexer_debug_fp8", st)
    return out
