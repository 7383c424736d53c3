"""CPU oracle for indexer top-k selection with paged slot mapping.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path. It shares
no code with the HIP library (see ``oracle_topk.c`` for the definition it
follows and its citation).

``topk_paged`` returns, per row, the selected logical positions and their
physical slots in (score descending, position ascending) order, padded with -1
to k. ``canonical`` reorders a result by position so that outputs in any order
(the GPU emits an unordered set) can be compared byte for byte.
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_topk.c")
_LIB = os.path.join(_HERE, "liboracle_topk.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``liboracle_topk.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.oracle_topk_paged_rows
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                      ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        _lib = lib
    return _lib


_ERRORS = {-1: "invalid argument", -2: "NaN inside a valid prefix",
           -3: "slot does not fit int32 or negative page", -4: "out of memory"}


def topk_paged(scores: np.ndarray, lengths: np.ndarray, block_table: np.ndarray,
               bt_row_stride: int, page_size: int, k: int, threads: int = 1):
    """Oracle top-k. Returns (idx, slots), each int32 [rows, k].

    ``threads`` > 1 runs disjoint row ranges concurrently (the C code releases
    nothing shared; ctypes drops the GIL during each call).
    """
    lib = _load()
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    rows, stride = scores.shape
    idx = np.empty((rows, k), np.int32)
    slots = np.empty((rows, k), np.int32)

    def run(lo: int, hi: int) -> int:
        return lib.oracle_topk_paged_rows(
            scores.ctypes.data, stride, lengths.ctypes.data, lo, hi,
            table.ctypes.data, int(bt_row_stride), int(page_size), int(k),
            idx.ctypes.data, slots.ctypes.data, k)

    if threads <= 1 or rows <= 1:
        rcs = [run(0, rows)]
    else:
        bounds = np.linspace(0, rows, min(threads, rows) + 1).astype(int)
        with _cf.ThreadPoolExecutor(len(bounds) - 1) as ex:
            rcs = list(ex.map(run, bounds[:-1], bounds[1:]))
    for rc in rcs:
        if rc != 0:
            raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")
    return idx, slots


def topk_workload(w, threads: int = 1):
    """Oracle on a ``synth.Workload``."""
    return topk_paged(w.scores, w.lengths, w.block_table, w.bt_row_stride,
                      w.page_size, w.k, threads=threads)


def canonical(idx: np.ndarray, slots: np.ndarray):
    """Sort each row's valid entries by position; -1 padding stays at the end.

    Entries equal to -1 sort last because positions are non-negative: the key
    maps -1 to the largest int64.
    """
    idx = np.asarray(idx)
    slots = np.asarray(slots)
    key = np.where(idx < 0, np.iinfo(np.int64).max, idx.astype(np.int64))
    order = np.argsort(key, axis=1, kind="stable")
    return (np.take_along_axis(idx, order, axis=1),
            np.take_along_axis(slots, order, axis=1))


def canonical_slots(slots: np.ndarray) -> np.ndarray:
    """Sort each row's slots ascending with -1 last (for slot-only outputs)."""
    s = np.asarray(slots).astype(np.int64)
    key = np.where(s < 0, np.iinfo(np.int64).max, s)
    return np.sort(key, axis=1)
