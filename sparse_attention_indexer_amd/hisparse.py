"""ctypes binding of the HiSparse top-k resolver (include/hisparse.h), in
``libsparse_topk.so``.

Argument marshalling only: classification, LRU victim choice, state updates
and the row copies from pinned host memory run in the library's HIP kernel.
There is no fallback: if the library is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes

import torch

from . import topk

DEVICE_HOT_FULL = 0x1000
DEVICE_BAD_INDEX = 0x2000


class hisparse_config(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("hot", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("row_bytes", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


_bound = False


def _lib():
    global _bound
    lib = topk.load_library()
    if not _bound:
        V, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        lib.hisparse_resolve.argtypes = [ctypes.POINTER(hisparse_config), U32, I32, V, I64, V, I64, V, I64, V, V, V,
                                         V, V, I64, V, I64, V, V, V]
        lib.hisparse_resolve.restype = ctypes.c_int
        _bound = True
    return lib


def hisparse_resolve(step: int, sel: torch.Tensor, block_table: torch.Tensor, host_table: torch.Tensor,
                     page_size: int, hot_rows: torch.Tensor, tag: torch.Tensor, stamp: torch.Tensor,
                     map_: torch.Tensor, kv: torch.Tensor, host_pool: torch.Tensor, rows_out: torch.Tensor,
                     status: torch.Tensor | None = None, stream=None) -> None:
    """One decode step for sel.shape[0] requests (see the header). host_pool is
    a pinned CPU uint8 tensor [host_rows, row_bytes]; kv a GPU uint8 tensor
    [kv_rows, row_bytes]; the state tensors are updated in place."""
    R, k = sel.shape
    hot = hot_rows.shape[1]
    max_ctx = map_.shape[1]
    for t, dt, name in ((sel, torch.int32, "sel"), (block_table, torch.int32, "block_table"),
                        (host_table, torch.int32, "host_table"), (hot_rows, torch.int64, "hot_rows"),
                        (tag, torch.int32, "tag"), (stamp, torch.int32, "stamp"), (map_, torch.int32, "map"),
                        (kv, torch.uint8, "kv"), (rows_out, torch.int64, "rows_out")):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous {dt} tensor on the GPU")
    if host_pool.dtype != torch.uint8 or host_pool.is_cuda or not host_pool.is_pinned() or \
            not host_pool.is_contiguous():
        raise TypeError("host_pool must be a contiguous pinned CPU uint8 tensor")
    if kv.dim() != 2 or host_pool.dim() != 2 or kv.shape[1] != host_pool.shape[1]:
        raise ValueError("kv and host_pool must be [rows, row_bytes] with the same row_bytes")
    if tuple(tag.shape) != (R, hot) or tuple(stamp.shape) != (R, hot) or map_.shape[0] != R or \
            tuple(rows_out.shape) != (R, k) or block_table.shape[0] != R or host_table.shape[0] != R:
        raise ValueError("state and table shapes do not match sel")
    cfg = hisparse_config(k, hot, int(page_size), max_ctx, kv.shape[1], (ctypes.c_int32 * 3)())
    st = _lib().hisparse_resolve(ctypes.byref(cfg), int(step), R, sel.data_ptr(), sel.stride(0),
                                 block_table.data_ptr(), block_table.stride(0), host_table.data_ptr(),
                                 host_table.stride(0), hot_rows.data_ptr(), tag.data_ptr(), stamp.data_ptr(),
                                 map_.data_ptr(), kv.data_ptr(), kv.shape[0], host_pool.data_ptr(),
                                 host_pool.shape[0], rows_out.data_ptr(),
                                 None if status is None else status.data_ptr(), topk._stream(stream))
    topk._check("hisparse_resolve", st)
