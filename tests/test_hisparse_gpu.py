"""GPU parity of the HiSparse top-k resolver against the oracle
(oracle/hisparse.py), through the C ABI: several requests over several decode
steps, the GPU and the oracle stepping in lock step from the same state.
Every output row, every state array (tags, stamps, position map) and every
hot KV row must be bit-identical after every step (integer work: exact)."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import hisparse as HS
from tests import _gpu

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    HAVE_GPU = False

pytestmark = pytest.mark.gpu
if not HAVE_GPU:
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_indexer_amd import hisparse as H  # noqa: E402


def scenario(R, ctx, ps, hot, k, row_bytes, seed, host_only=0.6):
    st = synth.Stream(seed, 61)
    pages = (ctx + ps - 1) // ps
    table = np.where(st.uniform(R * pages) < host_only, -1, st.permutation(R * pages)).astype(np.int32)
    table = table.reshape(R, pages)
    # a host pool of at most 512 pages (pages may share host copies: the data
    # only has to be the same on both sides); the KV tensor holds the hot rows
    # (resident rows are only named, never read or written)
    host_pages = min(R * pages, 512)
    host_table = st.below(R * pages, host_pages).astype(np.int32).reshape(R, pages)
    hot_rows = st.permutation(R * hot).astype(np.int64).reshape(R, hot)
    kv_rows = R * hot
    host_rows = host_pages * ps
    host = (st.u64(host_rows * row_bytes // 8).view(np.uint8)).reshape(host_rows, row_bytes).copy()
    return st, table, host_table, hot_rows, kv_rows, host


def selections(st, R, ctx, k, prev):
    sel = np.full((R, k), -1, np.int32)
    for r in range(R):
        pick = st.permutation(ctx)[:k]
        if prev is not None:
            old = prev[r][prev[r] >= 0][: k // 2]
            pick = np.unique(np.concatenate([old, pick]))[:k]
        n = min(k, pick.size) - (r == 1) * 3          # request 1 leaves a few -1 entries
        sel[r, :n] = pick[:n]
    return sel


def run_steps(R=4, ctx=20_000, ps=64, hot=512, k=256, row_bytes=656, steps=6, seed=1):
    st, table, host_table, hot_rows, kv_rows, host = scenario(R, ctx, ps, hot, k, row_bytes, seed)
    dev = torch.device("cuda:0")
    g = dict(table=torch.from_numpy(table).to(dev), host_table=torch.from_numpy(host_table).to(dev),
             hot_rows=torch.from_numpy(hot_rows).to(dev),
             tag=torch.full((R, hot), -1, dtype=torch.int32, device=dev),
             stamp=torch.zeros((R, hot), dtype=torch.int32, device=dev),
             map=torch.full((R, ctx), -1, dtype=torch.int32, device=dev),
             kv=torch.zeros((kv_rows, row_bytes), dtype=torch.uint8, device=dev),
             rows=torch.empty((R, k), dtype=torch.int64, device=dev),
             status=torch.zeros(1, dtype=torch.int32, device=dev))
    pool = torch.from_numpy(host).pin_memory()
    states = [HS.HotState.empty(hot, ctx) for _ in range(R)]
    kv = np.zeros((kv_rows, row_bytes), np.uint8)
    prev = None
    flags_seen = 0
    for step in range(1, steps + 1):
        sel = selections(st, R, ctx, k, prev)
        g["status"].zero_()
        H.hisparse_resolve(step, torch.from_numpy(sel).to(dev), g["table"], g["host_table"], ps, g["hot_rows"],
                           g["tag"], g["stamp"], g["map"], g["kv"], pool, g["rows"], g["status"])
        torch.cuda.synchronize()
        want_flags = 0
        for r in range(R):
            rows, f = HS.resolve(step, sel[r], table[r], host_table[r], ps, hot_rows[r], states[r], kv, host)
            want_flags |= f
            got = g["rows"][r].cpu().numpy()
            assert np.array_equal(got, rows), f"step {step} request {r}: rows differ at {np.flatnonzero(got != rows)[:5]}"
        tag, stamp, map_ = g["tag"].cpu().numpy(), g["stamp"].cpu().numpy().view(np.uint32), g["map"].cpu().numpy()
        for r in range(R):
            assert np.array_equal(tag[r], states[r].tag), f"step {step} request {r}: tags"
            assert np.array_equal(stamp[r], states[r].stamp), f"step {step} request {r}: stamps"
            assert np.array_equal(map_[r], states[r].map), f"step {step} request {r}: map"
        assert np.array_equal(g["kv"].cpu().numpy(), kv), f"step {step}: KV rows"
        status = int(g["status"].item())
        assert status == want_flags * H.DEVICE_HOT_FULL, (step, status, want_flags)
        flags_seen |= status
        prev = sel
    return flags_seen


def test_hisparse_steps_match_the_oracle():
    _gpu.say("[hisparse] 4 requests x 6 steps, k 256, hot 512")
    assert run_steps() == 0


def test_hisparse_full_size_decode_batch():
    _gpu.say("[hisparse] 8 requests x 4 steps, k 2048, hot 4096, 131072 context")
    run_steps(R=8, ctx=131_072, ps=64, hot=4096, k=2048, steps=4, seed=2)


def test_hisparse_hot_buffer_overflow_is_flagged():
    _gpu.say("[hisparse] hot buffer smaller than the misses")
    assert run_steps(R=2, ctx=3000, ps=16, hot=8, k=64, row_bytes=32, steps=3, seed=3) & H.DEVICE_HOT_FULL


def test_hisparse_rejects_pageable_host_memory():
    dev = torch.device("cuda:0")
    lib = H._lib()
    import ctypes
    cfg = H.hisparse_config(4, 8, 16, 64, 16, (ctypes.c_int32 * 3)())
    pageable = np.zeros((4, 16), np.uint8)
    d = torch.zeros(64, dtype=torch.int64, device=dev)
    st = lib.hisparse_resolve(ctypes.byref(cfg), 1, 1, d.data_ptr(), 4, d.data_ptr(), 4, d.data_ptr(), 4,
                              d.data_ptr(), d.data_ptr(), d.data_ptr(), d.data_ptr(), d.data_ptr(), 4,
                              pageable.ctypes.data, 4, d.data_ptr(), None, None)
    assert st == -1
