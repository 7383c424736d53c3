"""Independent checks of a top-k result, used to pin the oracle and to vet GPU output.

None of these re-run the oracle's algorithm (a full sort). They test what the
definition fixes: the rank-count characterisation of the selected set, the
invariants every correct answer satisfies, and the slot mapping through the
inverse of a page permutation.
"""
from __future__ import annotations

import numpy as np


def brute_force_select(row: np.ndarray, n: int, k: int) -> np.ndarray:
    """Positions i < n whose rank #{j: s_j > s_i or (s_j == s_i and j < i)} is < k.

    O(n^2) comparisons with IEEE semantics (so -0.0 == +0.0, -inf lowest).
    Returned in ascending position order.
    """
    s = np.asarray(row[:n], dtype=np.float32)
    if n == 0:
        return np.zeros(0, np.int64)
    pos = np.arange(n)
    gt = (s[None, :] > s[:, None]).sum(axis=1)
    eq_before = ((s[None, :] == s[:, None]) & (pos[None, :] < pos[:, None])).sum(axis=1)
    return pos[(gt + eq_before) < k]


def selected_positions(idx_row: np.ndarray) -> np.ndarray:
    v = np.asarray(idx_row)
    return np.sort(v[v >= 0]).astype(np.int64)


def invert_tables(block_table: np.ndarray, bt_row_stride: int, rows: int, page_size: int):
    """Per-row dict-free inverse: physical page -> logical page, as arrays.

    Tables are permutations of disjoint page sets, so each physical page has at
    most one logical page per row table.
    """
    inv = []
    for r in range(rows):
        t = block_table[0] if bt_row_stride == 0 else block_table[r]
        size = int(t.max()) + 1 if t.size else 1
        m = np.full(size, -1, np.int64)
        m[t.astype(np.int64)] = np.arange(t.size)
        inv.append(m)
    return inv


def check_row(row: np.ndarray, n: int, k: int, idx_row, slot_row, inv_table, page_size: int,
              label: str = "") -> None:
    """Assert every invariant of a correct answer for one row.

    ``idx_row`` may be None (slots only); then positions are recovered from
    the slots through the inverse table.
    """
    m = min(k, n)
    slot_row = np.asarray(slot_row).astype(np.int64)
    assert slot_row.shape == (k,), label
    valid = slot_row >= 0
    assert valid.sum() == m, f"{label}: {valid.sum()} entries, expected {m}"
    assert (slot_row[~valid] == -1).all(), f"{label}: padding is not -1"
    page = slot_row[valid] // page_size
    off = slot_row[valid] % page_size
    assert (page < inv_table.size).all(), f"{label}: slot outside the block table"
    logical = inv_table[page]
    assert (logical >= 0).all(), f"{label}: slot on a page the row does not own"
    from_slots = logical * page_size + off
    if idx_row is not None:
        idx_row = np.asarray(idx_row).astype(np.int64)
        assert ((idx_row >= 0) == valid).all(), f"{label}: idx/slot padding differ"
        assert (idx_row[valid] == from_slots).all(), f"{label}: slot is not the mapping of idx"
    pos = np.sort(from_slots)
    assert pos.size == np.unique(pos).size, f"{label}: repeated positions"
    if m == 0:
        return
    assert pos[0] >= 0 and pos[-1] < n, f"{label}: position outside [0, len)"
    s = np.asarray(row[:n], dtype=np.float32)
    chosen = np.zeros(n, bool)
    chosen[pos] = True
    if m < n:
        lo = s[chosen].min()
        hi = s[~chosen].max()
        assert lo >= hi, f"{label}: selected {lo} < unselected {hi}"
        # at the cut value the lowest positions win
        cut_sel = np.flatnonzero(chosen & (s == lo))
        cut_uns = np.flatnonzero(~chosen & (s == lo))
        if cut_uns.size:
            assert cut_sel.max() < cut_uns.min(), f"{label}: tie at the cut not lowest-index"
