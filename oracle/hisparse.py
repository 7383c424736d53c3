"""CPU oracle for the HiSparse top-k resolver: map each selected token of a
decode step to the KV-tensor row the sparse attention reads, keeping a
per-request LRU hot buffer filled from pinned host memory.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path. It shares
no code with the HIP library.

Source: the vllm.ai page "GLM 5.3 Optimizations, Part 1: Hybrid HiSparse
Offloading in vLLM", section "How it works" (mixed residency: the block table
holds real blocks and null placeholders; one fused kernel resolves the
top-K: resident tokens are read in place, hot tokens are read and their LRU
entry refreshed, a miss copies a single row from pinned host memory into an
LRU slot; the resolver hands out KV row IDs) and the hot-buffer size of 2x
top-K rows per request. The page gives no victim rule or data layout; the
readings implemented here:

* per request: a block-table row (physical page, or -1 for a page that lives
  only in host memory), a host block-table row (every page's host copy), H
  hot slots at given physical KV rows, and the hot state: tag[slot] (logical
  position held, -1 empty), stamp[slot] (step of last use, 0 never) and
  map[pos] (slot holding pos, -1 none);
* each call is one decode step with a stamp `step` larger than every stamp
  before it; the selected positions are distinct (a top-k output, -1 padded);
* a selected position p on a resident page reads row table[p / ps] * ps + p % ps;
  else, if map[p] >= 0, it reads hot_rows[map[p]] and stamp[map[p]] = step;
* else it is a miss. Misses are served in increasing position order; the
  victims are the slots not used in this step (stamp != step), least recently
  used first, ties (equal stamps: never-used slots) by lower slot index. Miss
  i takes victim i: the victim's old position is unmapped, the slot is tagged
  with p, stamped, and the host row (host_table[p / ps] * ps + p % ps of the
  host pool) is copied into KV row hot_rows[slot];
* if there are fewer victims than misses, the remaining misses (highest
  positions) get row -1 and a flag.
"""
from __future__ import annotations

import dataclasses

import numpy as np

HOT_FULL = 1   # flag: more misses than slots this step could evict


@dataclasses.dataclass
class HotState:
    tag: np.ndarray     # int32 [H]
    stamp: np.ndarray   # uint32 [H]
    map: np.ndarray     # int32 [max_ctx]

    @staticmethod
    def empty(hot: int, max_ctx: int) -> "HotState":
        return HotState(np.full(hot, -1, np.int32), np.zeros(hot, np.uint32), np.full(max_ctx, -1, np.int32))

    def copy(self) -> "HotState":
        return HotState(self.tag.copy(), self.stamp.copy(), self.map.copy())


def resolve(step: int, sel: np.ndarray, table: np.ndarray, host_table: np.ndarray, page_size: int,
            hot_rows: np.ndarray, st: HotState, kv: np.ndarray, host_pool: np.ndarray):
    """One request, one step. Mutates st and kv (rows [num_rows, row_bytes]
    uint8); host_pool is [host_rows, row_bytes] uint8. Returns (rows int64
    [len(sel)], flags)."""
    sel = np.asarray(sel, dtype=np.int64)
    rows = np.full(sel.shape, -1, np.int64)
    misses = []
    for j, p in enumerate(sel):
        if p < 0:
            continue
        page = int(table[p // page_size])
        if page >= 0:
            rows[j] = page * page_size + p % page_size
        elif st.map[p] >= 0:
            s = int(st.map[p])
            st.stamp[s] = step
            rows[j] = int(hot_rows[s])
        else:
            misses.append((int(p), j))
    misses.sort()
    cand = [s for s in range(len(st.tag)) if int(st.stamp[s]) != step]
    cand.sort(key=lambda s: (int(st.stamp[s]), s))
    flags = 0
    for i, (p, j) in enumerate(misses):
        if i >= len(cand):
            flags |= HOT_FULL
            continue
        s = cand[i]
        old = int(st.tag[s])
        if old >= 0:
            st.map[old] = -1
        st.tag[s] = p
        st.map[p] = s
        st.stamp[s] = step
        host_row = int(host_table[p // page_size]) * page_size + p % page_size
        kv[int(hot_rows[s])] = host_pool[host_row]
        rows[j] = int(hot_rows[s])
    return rows, flags
