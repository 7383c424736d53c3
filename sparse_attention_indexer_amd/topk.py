"""ctypes binding of ``libsparse_topk.so`` (the C ABI in include/sparse_topk.h).

Argument marshalling only: every step of planning, selection and slot mapping
runs in the library's HIP kernels. torch supplies device memory and the
current stream. There is no fallback: if the library is not built, or its
device calls fail, these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_topk.so")

TOPK_OK = 0
TOPK_ERR_INVALID_ARG = -1
TOPK_ERR_BUFFER_TOO_SMALL = -2
TOPK_ERR_UNSUPPORTED = -3
TOPK_ERR_HIP = -4
TOPK_ERR_DEVICE = -5

PATH_AUTO, PATH_REGISTER, PATH_SINGLE, PATH_MULTI = 0, 1, 2, 3
PATHS = {"auto": PATH_AUTO, "register": PATH_REGISTER, "single": PATH_SINGLE, "multi": PATH_MULTI}

DEVICE_SPIN_TIMEOUT, DEVICE_PLAN_MISMATCH, DEVICE_BAD_LENGTH, DEVICE_INTERNAL = 1, 2, 4, 8


class topk_config(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("max_rows", ctypes.c_int32), ("max_len", ctypes.c_int64),
                ("force_path", ctypes.c_int32), ("wg_per_row", ctypes.c_int32),
                ("cand_capacity", ctypes.c_int32), ("min_chunk", ctypes.c_int32),
                ("spin_limit", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


class TopKError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_lib = None


def load_library():
    """Load the in-tree HIP library, or raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_attention_indexer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, I64, V = (ctypes.POINTER(topk_config), ctypes.c_size_t, ctypes.c_int32,
                         ctypes.c_int64, ctypes.c_void_p)
    sigs = {
        "topk_query_sizes": [P, ctypes.POINTER(S), ctypes.POINTER(S)],
        "topk_workspace_init": [V, S, V],
        "topk_plan": [P, V, I32, V, S, V],
        "topk_select_paged": [P, V, V, I64, V, I32, V, I64, I32, V, V, I64, V, S, V],
        "topk_select_paged_timed": [P, V, V, I64, V, I32, V, I64, I32, V, V, I64, V, S, V, V, V],
        "topk_read_status": [V, S, ctypes.POINTER(I32), V],
        "topk_debug_keys": [V, I64, V, V, V],
        "topk_debug_stream_read": [V, I64, V, V, V, V],
        "topk_debug_histogram": [V, I64, V, I32, I32, V, V, V],
        "topk_select_paged_noalloc": [P, V, I64, V, I32, V, I64, I32, V, V, I64, V, V],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.topk_register_capacity.argtypes = []
    lib.topk_register_capacity.restype = ctypes.c_int64
    lib.topk_stream_read_groups.argtypes = []
    lib.topk_stream_read_groups.restype = ctypes.c_int32
    lib.topk_status_string.argtypes = [ctypes.c_int]
    lib.topk_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, st: int) -> None:
    if st != TOPK_OK:
        msg = load_library().topk_status_string(st).decode()
        raise TopKError(fn, st, msg)


def make_config(k: int, max_rows: int, max_len: int, force_path: int | str = PATH_AUTO,
                wg_per_row: int = 0, cand_capacity: int = 0, min_chunk: int = 0,
                spin_limit: int = 0) -> topk_config:
    if isinstance(force_path, str):
        force_path = PATHS[force_path]
    return topk_config(int(k), int(max_rows), int(max_len), int(force_path), int(wg_per_row),
                       int(cand_capacity), int(min_chunk), int(spin_limit), (ctypes.c_int32 * 3)())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} tensor on the GPU")


def _check_layout(lengths: torch.Tensor, block_table: torch.Tensor | None = None) -> None:
    """The library reads lengths as a dense int32 array and each block-table
    row as consecutive entries; a strided view would be read as other data."""
    if not lengths.is_contiguous():
        raise ValueError("lengths must be contiguous")
    if block_table is not None and block_table.dim() > 0 and block_table.stride(-1) != 1:
        raise ValueError("block_table must have unit stride along pages")


# --- functions with the C names ------------------------------------------------

def topk_query_sizes(cfg: topk_config) -> tuple[int, int]:
    plan, ws = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("topk_query_sizes", load_library().topk_query_sizes(ctypes.byref(cfg), ctypes.byref(plan),
                                                               ctypes.byref(ws)))
    return plan.value, ws.value


def topk_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    _check("topk_workspace_init", load_library().topk_workspace_init(
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))


def topk_plan(cfg: topk_config, lengths: torch.Tensor, plan: torch.Tensor, stream=None) -> None:
    _check_layout(lengths)
    _need(lengths, torch.int32, "lengths")
    _check("topk_plan", load_library().topk_plan(
        ctypes.byref(cfg), lengths.data_ptr(), lengths.numel(), plan.data_ptr(),
        plan.numel() * plan.element_size(), _stream(stream)))


def _select_args(cfg, plan, scores, lengths, block_table, bt_row_stride, page_size, out_slots, out_indices,
                 workspace, stream):
    _check_layout(lengths, block_table)
    _need(scores, torch.float32, "scores")
    _need(lengths, torch.int32, "lengths")
    _need(block_table, torch.int32, "block_table")
    _need(out_slots, torch.int32, "out_slots")
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be 2-D with unit stride along positions")
    if out_slots.dim() != 2 or out_slots.stride(1) != 1:
        raise ValueError("out_slots must be 2-D with unit inner stride")
    if out_indices is not None:
        _need(out_indices, torch.int32, "out_indices")
        if out_indices.stride() != out_slots.stride():
            raise ValueError("out_indices must have out_slots' strides")
    rows = lengths.numel()
    if scores.shape[0] < rows or out_slots.shape[0] < rows:
        raise ValueError("scores and out_slots need a row per length")
    return (ctypes.byref(cfg), _ptr(plan), scores.data_ptr(), scores.stride(0), lengths.data_ptr(), rows,
            block_table.data_ptr(), int(bt_row_stride), int(page_size), out_slots.data_ptr(),
            _ptr(out_indices), out_slots.stride(0), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))


def topk_select_paged(cfg: topk_config, plan: torch.Tensor, scores: torch.Tensor, lengths: torch.Tensor,
                      block_table: torch.Tensor, bt_row_stride: int, page_size: int,
                      out_slots: torch.Tensor, out_indices: torch.Tensor | None,
                      workspace: torch.Tensor, stream=None) -> None:
    args = _select_args(cfg, plan, scores, lengths, block_table, bt_row_stride, page_size, out_slots,
                        out_indices, workspace, stream)
    _check("topk_select_paged", load_library().topk_select_paged(*args))


def topk_select_paged_noalloc(cfg: topk_config, scores: torch.Tensor, lengths: torch.Tensor,
                              block_table: torch.Tensor, bt_row_stride: int, page_size: int,
                              out_slots: torch.Tensor, out_indices: torch.Tensor | None,
                              device_status: torch.Tensor | None = None, stream=None) -> None:
    """topk_select_paged with no plan or workspace: the library's own device
    array holds the cross-workgroup state (batches planned in the kernel)."""
    args = _select_args(cfg, None, scores, lengths, block_table, bt_row_stride, page_size, out_slots,
                        out_indices, None, stream)
    if device_status is not None:
        _need(device_status, torch.int32, "device_status")
    # (cfg, scores, stride, lengths, rows, table, bt stride, page size, slots, indices, out stride)
    _check("topk_select_paged_noalloc", load_library().topk_select_paged_noalloc(
        *args[0:1], *args[2:12], _ptr(device_status), args[14]))


def _event_handle(ev: "torch.cuda.Event") -> int:
    """The hipEvent_t behind a torch event (torch creates it on first record)."""
    if not ev.cuda_event:
        ev.record()
    return int(ev.cuda_event)


def topk_select_paged_timed(cfg: topk_config, plan: torch.Tensor, scores: torch.Tensor, lengths: torch.Tensor,
                            block_table: torch.Tensor, bt_row_stride: int, page_size: int,
                            out_slots: torch.Tensor, out_indices: torch.Tensor | None,
                            workspace: torch.Tensor, start: "torch.cuda.Event", stop: "torch.cuda.Event",
                            stream=None) -> None:
    """topk_select_paged whose kernel records its own start and end into two
    timing-enabled torch events (read them with start.elapsed_time(stop))."""
    args = _select_args(cfg, plan, scores, lengths, block_table, bt_row_stride, page_size, out_slots,
                        out_indices, workspace, stream)
    _check("topk_select_paged_timed", load_library().topk_select_paged_timed(
        *args, _event_handle(start), _event_handle(stop)))


def topk_read_status(workspace: torch.Tensor, stream=None) -> int:
    v = ctypes.c_int32(0)
    st = load_library().topk_read_status(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                         ctypes.byref(v), _stream(stream))
    if st not in (TOPK_OK, TOPK_ERR_DEVICE):
        _check("topk_read_status", st)
    return v.value


def topk_register_capacity() -> int:
    return int(load_library().topk_register_capacity())


def topk_debug_keys(x: torch.Tensor, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    _need(x, torch.float32, "x")
    x = x.contiguous()
    bins = torch.empty(x.numel(), dtype=torch.int32, device=x.device)
    keys = torch.empty(x.numel(), dtype=torch.int32, device=x.device)
    _check("topk_debug_keys", load_library().topk_debug_keys(x.data_ptr(), x.numel(), bins.data_ptr(),
                                                             keys.data_ptr(), _stream(stream)))
    return bins, keys


def topk_debug_histogram(scores: torch.Tensor, lengths: torch.Tensor, k: int, stream=None):
    """The selection kernel's coarse histogram (int32 [rows, 1024], ordered
    bins) and threshold (int32 [rows, 3]: b*, above, count) of each row."""
    _check_layout(lengths)
    _need(scores, torch.float32, "scores")
    _need(lengths, torch.int32, "lengths")
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be 2-D with unit stride along positions")
    rows = lengths.numel()
    hist = torch.empty((rows, 1024), dtype=torch.int32, device=scores.device)
    thr = torch.empty((rows, 3), dtype=torch.int32, device=scores.device)
    _check("topk_debug_histogram", load_library().topk_debug_histogram(
        scores.data_ptr(), scores.stride(0), lengths.data_ptr(), rows, int(k), hist.data_ptr(),
        thr.data_ptr(), _stream(stream)))
    return hist, thr


def topk_debug_stream_read(x: torch.Tensor, out: torch.Tensor | None = None, stream=None,
                           events=None) -> torch.Tensor:
    """One streaming read of ``x`` (float32, contiguous, 16-byte aligned) with
    the selection kernel's load pattern; returns the per-workgroup partial sums.
    ``events``: optional (start, stop) torch.cuda.Event pair that records the
    kernel's own start and end."""
    _need(x, torch.float32, "x")
    lib = load_library()
    if out is None:
        out = torch.empty(int(lib.topk_stream_read_groups()), dtype=torch.float32, device=x.device)
    ev = (None, None) if events is None else (_event_handle(events[0]), _event_handle(events[1]))
    _check("topk_debug_stream_read", lib.topk_debug_stream_read(x.data_ptr(), x.numel(), out.data_ptr(),
                                                                _stream(stream), ev[0], ev[1]))
    return out


# --- convenience wrapper ----------------------------------------------------------

class TopK:
    """Owns a plan and a workspace sized for one configuration on one device."""

    def __init__(self, k: int, max_rows: int, max_len: int, *, force_path: int | str = PATH_AUTO,
                 wg_per_row: int = 0, cand_capacity: int = 0, min_chunk: int = 0, spin_limit: int = 0,
                 device=None):
        self.device = torch.device("cuda" if device is None else device)
        self.cfg = make_config(k, max_rows, max_len, force_path, wg_per_row, cand_capacity, min_chunk,
                               spin_limit)
        with torch.cuda.device(self.device):
            plan_bytes, ws_bytes = topk_query_sizes(self.cfg)
            self.plan_buf = torch.zeros((plan_bytes + 15) // 16 * 4, dtype=torch.int32, device=self.device)
            self.workspace = torch.empty((ws_bytes + 15) // 16 * 4, dtype=torch.int32, device=self.device)
            topk_workspace_init(self.workspace)
        self.k = int(k)

    def plan(self, lengths: torch.Tensor, stream=None) -> None:
        topk_plan(self.cfg, lengths, self.plan_buf, stream)

    def select(self, scores: torch.Tensor, lengths: torch.Tensor, block_table: torch.Tensor,
               bt_row_stride: int, page_size: int, *, out_slots: torch.Tensor | None = None,
               out_indices: torch.Tensor | None = None, with_indices: bool = True, stream=None,
               events: tuple | None = None):
        rows = lengths.numel()
        if out_slots is None:
            out_slots = torch.empty((rows, self.k), dtype=torch.int32, device=scores.device)
        if out_indices is None and with_indices:
            out_indices = torch.empty_like(out_slots)
        if events is None:
            topk_select_paged(self.cfg, self.plan_buf, scores, lengths, block_table, bt_row_stride, page_size,
                              out_slots, out_indices, self.workspace, stream)
        else:
            topk_select_paged_timed(self.cfg, self.plan_buf, scores, lengths, block_table, bt_row_stride,
                                    page_size, out_slots, out_indices, self.workspace, events[0], events[1],
                                    stream)
        return out_slots, out_indices

    def status(self, stream=None) -> int:
        return topk_read_status(self.workspace, stream)
