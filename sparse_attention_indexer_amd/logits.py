"""ctypes binding of the indexer's MQA logits (include/indexer_logits.h), in
``libsparse_topk.so``.

Argument marshalling only: the FP8 dot products, ReLU, head-gate weighting
and key scaling run in the library's HIP kernel (matrix cores). There is no
fallback: if the library is missing or a call fails, these functions raise.
"""
from __future__ import annotations

import ctypes

import torch

from . import topk

MAX_QROWS = 512
_bound = False


def _lib():
    global _bound
    lib = topk.load_library()
    if not _bound:
        V, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.indexer_mqa_logits.argtypes = [V, V, I32, I32, V, V, I64, V, I32, V, I32, V, I64, V, V]
        lib.indexer_mqa_logits.restype = ctypes.c_int
        _bound = True
    return lib


def indexer_mqa_logits(q_codes: torch.Tensor, w: torch.Tensor, k_fp8: torch.Tensor, k_scale: torch.Tensor,
                       block_table_row: torch.Tensor, page_size: int, lengths: torch.Tensor, max_len: int,
                       out: torch.Tensor, status: torch.Tensor | None = None, stream=None) -> None:
    """Scores of q_codes [T, H, 128] (uint8) against the key cache k_fp8
    [slots, 128] / k_scale [slots] into out [T, >= max_len] (float32); only
    out[t, :min(lengths[t], max_len)] is written."""
    for t, dt, name in ((q_codes, torch.uint8, "q_codes"), (w, torch.float32, "w"), (k_fp8, torch.uint8, "k_fp8"),
                        (k_scale, torch.float32, "k_scale"), (block_table_row, torch.int32, "block_table_row"),
                        (lengths, torch.int32, "lengths"), (out, torch.float32, "out")):
        if t.dtype != dt or not t.is_cuda:
            raise TypeError(f"{name} must be a {dt} tensor on the GPU")
    if q_codes.dim() != 3 or q_codes.shape[2] != 128 or not q_codes.is_contiguous():
        raise ValueError("q_codes must be a contiguous [tokens, heads, 128] tensor")
    T, H = q_codes.shape[0], q_codes.shape[1]
    if tuple(w.shape) != (T, H) or not w.is_contiguous() or lengths.numel() != T or not lengths.is_contiguous():
        raise ValueError("w must be [tokens, heads] and lengths [tokens], contiguous")
    if k_fp8.dim() != 2 or k_fp8.shape[1] != 128 or not k_fp8.is_contiguous() or k_scale.numel() != k_fp8.shape[0]:
        raise ValueError("k_fp8 must be a contiguous [slots, 128] tensor and k_scale [slots]")
    if out.dim() != 2 or out.shape[0] != T or out.stride(1) != 1 or out.shape[1] < max_len:
        raise ValueError("out must be [tokens, >= max_len] with unit inner stride")
    if block_table_row.dim() != 1 or not block_table_row.is_contiguous():
        raise ValueError("block_table_row must be one contiguous table row")
    st = _lib().indexer_mqa_logits(q_codes.data_ptr(), w.data_ptr(), T, H, k_fp8.data_ptr(), k_scale.data_ptr(),
                                   k_fp8.shape[0], block_table_row.data_ptr(), int(page_size), lengths.data_ptr(),
                                   int(max_len), out.data_ptr(), out.stride(0),
                                   None if status is None else status.data_ptr(), topk._stream(stream))
    topk._check("indexer_mqa_logits", st)
