"""Pins for the CPU oracle (no GPU).

The oracle is a full sort; each test below checks it against something other
than a sort written the same way: brute-force rank counting, an exhaustive
search over subsets, numpy's stable argsort, argmax, closed forms of the
adversarial rows, hand-worked tie cases, and the inverse page permutation.
``test_planted_mistakes`` compiles mutated copies of the oracle and checks that
these pins reject every one of them.
"""
from __future__ import annotations

import ctypes
import itertools
import os
import subprocess
import sys

import numpy as np
import pytest

import synth
from tests import _checks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "ties.txt")


def _parse_float(tok: str) -> float:
    special = {"inf": np.inf, "-inf": -np.inf, "-0": -0.0}
    return special[tok] if tok in special else float(tok)


def load_golden():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, k, n, scores, expect = [p.strip() for p in line.split("|")]
            row = np.array([_parse_float(t) for t in scores.split()], np.float32)
            exp = np.array([int(t) for t in expect.split()], np.int64)
            cases.append((name, int(k), int(n), row, exp))
    return cases


def run_one_row(oracle_mod, row, n, k, ps=64, table=None):
    row = np.asarray(row, np.float32)[None, :]
    pages = max(1, (row.shape[1] + ps - 1) // ps)
    if table is None:
        table = np.arange(pages, dtype=np.int32)[None, :]
    idx, slots = oracle_mod.topk_paged(row, np.array([n], np.int32), table, 0, ps, k)
    return idx[0], slots[0]


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c[0])
def test_golden_ties(oracle_mod, case):
    name, k, n, row, exp = case
    idx, slots = run_one_row(oracle_mod, row, n, k)
    np.testing.assert_array_equal(_checks.selected_positions(idx), exp)
    # identity table: slot == position
    np.testing.assert_array_equal(idx, slots)
    assert (idx[len(exp):] == -1).all()


def test_brute_force_rank_count(oracle_mod):
    for trial in range(300):
        st = synth.Stream(1234, trial)
        n = int(st.below(1, 40)[0])
        alpha = np.array([0.0, -0.0, 1.5, -2.0, -np.inf, 1.5, 3.25], np.float32)
        choice = st.below(max(n, 1), 2 + int(st.below(1, 5)[0]))
        row = alpha[choice][:n] if n else np.zeros(0, np.float32)
        row = np.concatenate([row, np.full(3, 7e30, np.float32)])  # junk past len
        for k in range(1, n + 3):
            idx, _ = run_one_row(oracle_mod, row, n, k)
            got = _checks.selected_positions(idx)
            np.testing.assert_array_equal(got, _checks.brute_force_select(row, n, k),
                                          err_msg=f"trial {trial} k {k}")


def test_brute_force_medium(oracle_mod):
    w = synth.random_case(7, rows=6, max_len=3000, alphabet=40, special=True)
    idx, slots = oracle_mod.topk_workload(w)
    for r in range(w.rows):
        n = int(w.lengths[r])
        np.testing.assert_array_equal(_checks.selected_positions(idx[r]),
                                      _checks.brute_force_select(w.scores[r], n, w.k))


def _exhaustive_best(row, n, k):
    """Search all subsets of size min(k, n): maximise the descending score
    vector lexicographically, then minimise the ascending position vector."""
    m = min(k, n)
    best = None
    for sub in itertools.combinations(range(n), m):
        vals = tuple(sorted((float(row[i]) for i in sub), reverse=True))
        key = (tuple(-v for v in vals), sub)     # combinations are ascending
        if best is None or key < best[0]:
            best = (key, sub)
    return np.array(best[1] if best else (), np.int64)


def test_exhaustive_subsets(oracle_mod):
    for trial in range(60):
        st = synth.Stream(99, trial)
        n = 1 + int(st.below(1, 9)[0])
        alpha = np.array([0.0, -0.0, 2.0, -1.0, -np.inf, 2.0], np.float32)
        row = alpha[st.below(n, 6)]
        for k in range(1, n + 2):
            idx, _ = run_one_row(oracle_mod, row, n, k)
            np.testing.assert_array_equal(_checks.selected_positions(idx),
                                          _exhaustive_best(row, n, k))


def test_numpy_stable_argsort(oracle_mod):
    """Stable argsort of the negated scores orders by (score desc, position asc):
    negation keeps -0.0 == +0.0, so equal scores keep position order."""
    for seed, alpha in ((3, 0), (4, 25), (5, 3)):
        w = synth.random_case(seed, rows=5, max_len=20_000, alphabet=alpha, special=True)
        idx, _ = oracle_mod.topk_workload(w)
        for r in range(w.rows):
            n = int(w.lengths[r])
            ref = np.argsort(-w.scores[r, :n], kind="stable")[: w.k]
            np.testing.assert_array_equal(idx[r, : ref.size], ref)
            assert (idx[r, ref.size:] == -1).all()


def test_c1_against_argsort(oracle_mod):
    w = synth.make_config(1)
    idx, slots = oracle_mod.topk_workload(w)
    inv = _checks.invert_tables(w.block_table, w.bt_row_stride, w.rows, w.page_size)
    for r in range(w.rows):
        ref = np.argsort(-w.scores[r], kind="stable")[: w.k]
        np.testing.assert_array_equal(idx[r], ref)
        _checks.check_row(w.scores[r], int(w.lengths[r]), w.k, idx[r], slots[r], inv[r],
                          w.page_size, f"c1 row {r}")


def test_k1_is_first_argmax(oracle_mod):
    w = synth.random_case(11, rows=20, max_len=500, alphabet=6, special=True, k=1)
    idx, _ = oracle_mod.topk_workload(w)
    for r in range(w.rows):
        n = int(w.lengths[r])
        if n == 0:
            assert idx[r, 0] == -1
        else:
            assert idx[r, 0] == int(np.argmax(w.scores[r, :n]))


@pytest.mark.slow
def test_c5_closed_forms(oracle_mod):
    w = synth.make_config(5)
    idx, slots = oracle_mod.topk_workload(w, threads=8)
    inv = _checks.invert_tables(w.block_table, w.bt_row_stride, w.rows, w.page_size)
    first = np.arange(w.k)
    for r in range(w.rows):
        got = _checks.selected_positions(idx[r])
        g = r // 64
        if g in (0, 3):
            # all-equal rows and sorted-descending rows: the first k positions
            np.testing.assert_array_equal(got, first, err_msg=f"row {r}")
        elif g == 1:
            # 16 values: the top value occurs far more than k times, so the
            # answer is the k lowest positions holding the row maximum
            top = np.flatnonzero(w.scores[r] == w.scores[r].max())
            assert top.size >= w.k
            np.testing.assert_array_equal(got, top[: w.k], err_msg=f"row {r}")
        else:
            np.testing.assert_array_equal(
                got, np.sort(np.argsort(-w.scores[r], kind="stable")[: w.k]))
        _checks.check_row(w.scores[r], int(w.lengths[r]), w.k, idx[r], slots[r], inv[r],
                          w.page_size, f"c5 row {r}")


def test_c4_short_rows_return_all(oracle_mod):
    w = synth.make_config(4)
    short = np.flatnonzero(w.lengths <= w.k)
    assert short.size > 0
    sub = w.scores[short]
    idx, _ = oracle_mod.topk_paged(sub, w.lengths[short], w.block_table[short],
                                   w.bt_row_stride, w.page_size, w.k)
    for j, r in enumerate(short):
        np.testing.assert_array_equal(_checks.selected_positions(idx[j]),
                                      np.arange(w.lengths[r]))


def test_slot_page_boundaries(oracle_mod):
    # table [5, 2, 9]: position 63 is the last slot of page 5, 64 the first of page 2
    row = np.zeros(192, np.float32)
    row[[63, 64, 191]] = [3.0, 2.0, 1.0]
    table = np.array([[5, 2, 9]], np.int32)
    idx, slots = run_one_row(oracle_mod, row, 192, 3, ps=64, table=table)
    assert list(idx) == [63, 64, 191]
    assert list(slots) == [5 * 64 + 63, 2 * 64, 9 * 64 + 63]


@pytest.mark.parametrize("ps", [1, 16, 64, 128])
@pytest.mark.parametrize("shared", [True, False])
def test_slots_invert_to_positions(oracle_mod, ps, shared):
    w = synth.random_case(21 + ps, rows=4, max_len=5000, page_size=ps, shared_table=shared,
                          alphabet=30, k=700)
    idx, slots = oracle_mod.topk_workload(w)
    inv = _checks.invert_tables(w.block_table, w.bt_row_stride, w.rows, ps)
    for r in range(w.rows):
        _checks.check_row(w.scores[r], int(w.lengths[r]), w.k, idx[r], slots[r], inv[r], ps,
                          f"ps {ps} row {r}")


def test_nan_rejected_only_inside_prefix(oracle_mod):
    row = np.array([1.0, np.nan, 2.0], np.float32)
    with pytest.raises(ValueError):
        run_one_row(oracle_mod, row, 3, 1)
    idx, _ = run_one_row(oracle_mod, row, 1, 1)     # NaN lies past len
    assert idx[0] == 0


def test_invariants_on_generated_configs(oracle_mod):
    for i in (1, 2, 4):
        w = synth.make_config(i)
        idx, slots = oracle_mod.topk_workload(w, threads=8)
        inv = _checks.invert_tables(w.block_table, w.bt_row_stride, w.rows, w.page_size)
        for r in range(w.rows):
            _checks.check_row(w.scores[r], int(w.lengths[r]), w.k, idx[r], slots[r], inv[r],
                              w.page_size, f"c{i} row {r}")


def test_canonical_sorts_by_position(oracle_mod):
    idx = np.array([[5, 2, 9, -1, -1]], np.int32)
    slots = np.array([[50, 20, 90, -1, -1]], np.int32)
    ci, cs = oracle_mod.canonical(idx, slots)
    assert ci.tolist() == [[2, 5, 9, -1, -1]] and cs.tolist() == [[20, 50, 90, -1, -1]]


# Hand-worked rows for the two comparators: each row is reordered on its own,
# slots travel with their positions, and -1 padding stays at the end. Row 1's
# slots are not ordered like its positions (the table is a permutation), so a
# comparator that sorted slots by slot value, or sorted across rows, or moved
# -1 to the front, gives a different answer.
_CANON_IDX = np.array([[7, 0, 3, -1, -1],
                       [1, 9, 4, 2, -1],
                       [-1, -1, -1, -1, -1]], np.int32)
_CANON_SLOTS = np.array([[455, 128, 195, -1, -1],
                         [65, 9, 388, 130, -1],
                         [-1, -1, -1, -1, -1]], np.int32)
_CANON_WANT_IDX = [[0, 3, 7, -1, -1], [1, 2, 4, 9, -1], [-1, -1, -1, -1, -1]]
_CANON_WANT_SLOTS = [[128, 195, 455, -1, -1], [65, 130, 388, 9, -1], [-1, -1, -1, -1, -1]]
# slot-only comparison: each row's slots ascending, -1 (as the int64 maximum) last
_BIG = int(np.iinfo(np.int64).max)
_CANON_WANT_SLOT_ONLY = [[128, 195, 455, _BIG, _BIG], [9, 65, 130, 388, _BIG], [_BIG] * 5]


def _canonical_pins_pass(canonical, canonical_slots) -> bool:
    ci, cs = canonical(_CANON_IDX, _CANON_SLOTS)
    if np.asarray(ci).tolist() != _CANON_WANT_IDX or np.asarray(cs).tolist() != _CANON_WANT_SLOTS:
        return False
    return np.asarray(canonical_slots(_CANON_SLOTS)).tolist() == _CANON_WANT_SLOT_ONLY


def test_canonical_multi_row_hand_worked(oracle_mod):
    assert _canonical_pins_pass(oracle_mod.canonical, oracle_mod.canonical_slots)


def test_canonical_slots_keeps_rows_apart(oracle_mod):
    """Two outputs of the same row set in different orders compare equal; a
    slot moved to another row does not."""
    a = np.array([[3, 1, 2, -1], [8, 6, -1, -1]], np.int32)
    b = np.array([[2, 3, 1, -1], [-1, 6, 8, -1]], np.int32)
    c = np.array([[3, 1, 8, -1], [2, 6, -1, -1]], np.int32)
    sa, sb, sc = (oracle_mod.canonical_slots(x) for x in (a, b, c))
    assert np.array_equal(sa, sb)
    assert not np.array_equal(sa, sc)


def _canon_slots_axis0(slots):
    s = np.asarray(slots).astype(np.int64)
    return np.sort(np.where(s < 0, np.iinfo(np.int64).max, s), axis=0)


def _canon_slots_minus_one_first(slots):
    return np.sort(np.asarray(slots).astype(np.int64), axis=1)


def _canon_by_slot(idx, slots):
    order = np.argsort(np.where(np.asarray(slots) < 0, np.iinfo(np.int64).max, slots), axis=1, kind="stable")
    return np.take_along_axis(idx, order, axis=1), np.take_along_axis(slots, order, axis=1)


def _canon_slots_unmoved(idx, slots):
    key = np.where(idx < 0, np.iinfo(np.int64).max, idx.astype(np.int64))
    return np.sort(key, axis=1).astype(np.int32), np.asarray(slots)


@pytest.mark.parametrize("mistake", ["slots_axis0", "slots_minus_one_first", "canon_by_slot",
                                     "canon_slots_unmoved"])
def test_canonical_planted_mistakes(oracle_mod, mistake):
    canonical, canonical_slots = oracle_mod.canonical, oracle_mod.canonical_slots
    if mistake == "slots_axis0":
        canonical_slots = _canon_slots_axis0
    elif mistake == "slots_minus_one_first":
        canonical_slots = _canon_slots_minus_one_first
    elif mistake == "canon_by_slot":
        canonical = _canon_by_slot
    else:
        canonical = _canon_slots_unmoved
    assert not _canonical_pins_pass(canonical, canonical_slots)


# --- planted mistakes: each mutated copy of the oracle must fail a pin --------

MUTATIONS = {
    "tie_high_index_first": ("return (a->pos > b->pos) - (a->pos < b->pos);",
                             "return (a->pos < b->pos) - (a->pos > b->pos);"),
    "ascending_scores": ("if (a->score > b->score) return -1;",
                         "if (a->score > b->score) return 1;"),
    "offset_dropped": ("(int64_t)(idx % page_size)", "(int64_t)0"),
    "page_off_by_one": ("table[idx / page_size]", "table[(idx + 1) / page_size]"),
    "no_padding_rule": ("const int32_t m = n < k ? n : k;", "const int32_t m = k;"),
    "reads_past_len": ("const int32_t n = lengths[r];",
                       "const int32_t n = (int32_t)score_stride;"),
    "truncates_one_short": ("const int32_t m = n < k ? n : k;",
                            "const int32_t m = (n < k ? n : k) - (n > 1);"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "oracle_topk.c")).read()
    assert src.count(old) == 1, name
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-o", str(so), str(path), "-lm"])
    return str(so)


class _MutantOracle:
    def __init__(self, lib):
        self.lib = lib
        f = lib.oracle_topk_paged_rows
        f.restype = ctypes.c_int

    def topk_paged(self, scores, lengths, table, bt_stride, ps, k):
        scores = np.ascontiguousarray(scores, np.float32)
        lengths = np.ascontiguousarray(lengths, np.int32)
        table = np.ascontiguousarray(table, np.int32)
        rows, stride = scores.shape
        idx = np.full((rows, k), -7, np.int32)
        slots = np.full((rows, k), -7, np.int32)
        rc = self.lib.oracle_topk_paged_rows(
            ctypes.c_void_p(scores.ctypes.data), ctypes.c_int64(stride),
            ctypes.c_void_p(lengths.ctypes.data), ctypes.c_int32(0), ctypes.c_int32(rows),
            ctypes.c_void_p(table.ctypes.data), ctypes.c_int64(bt_stride),
            ctypes.c_int32(ps), ctypes.c_int32(k), ctypes.c_void_p(idx.ctypes.data),
            ctypes.c_void_p(slots.ctypes.data), ctypes.c_int64(k))
        if rc != 0:
            raise ValueError(rc)
        return idx, slots


def _pins_pass(mod) -> bool:
    """Run a compact subset of the pins against ``mod``; False on any failure."""
    try:
        for name, k, n, row, exp in load_golden():
            pages = max(1, (row.size + 63) // 64)
            idx, slots = mod.topk_paged(row[None, :], np.array([n], np.int32),
                                        np.arange(pages, dtype=np.int32)[None, :], 0, 64, k)
            if not np.array_equal(_checks.selected_positions(idx[0]), exp):
                return False
            if not ((idx[0][exp.size:] == -1).all() and np.array_equal(idx[0], slots[0])):
                return False
        row = np.zeros(192, np.float32)
        row[[63, 64, 191]] = [3.0, 2.0, 1.0]
        idx, slots = mod.topk_paged(row[None, :], np.array([192], np.int32),
                                    np.array([[5, 2, 9]], np.int32), 0, 64, 3)
        if list(slots[0]) != [383, 128, 639]:
            return False
        w = synth.random_case(7, rows=4, max_len=600, alphabet=12, special=True, k=50)
        idx, slots = mod.topk_paged(w.scores, w.lengths, w.block_table, w.bt_row_stride,
                                    w.page_size, w.k)
        inv = _checks.invert_tables(w.block_table, w.bt_row_stride, w.rows, w.page_size)
        for r in range(w.rows):
            n = int(w.lengths[r])
            if not np.array_equal(_checks.selected_positions(idx[r]),
                                  _checks.brute_force_select(w.scores[r], n, w.k)):
                return False
            _checks.check_row(w.scores[r], n, w.k, idx[r], slots[r], inv[r], w.page_size)
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def test_pins_accept_real_oracle(oracle_mod):
    assert _pins_pass(oracle_mod)


# Run in a child process: several mutants read or write out of bounds (a
# padding rule dropped reads past the sorted pairs, a length ignored overruns
# the pair buffer), and the resulting crash must not take the test run down.
# Exit status 0 means the pins accepted the mutant; 3 that they rejected it;
# a crash also counts as rejected, since the pins could not pass.
_CHILD = """
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from tests import test_oracle as t
mutant = t._MutantOracle(ctypes.CDLL(sys.argv[2]))
sys.exit(0 if t._pins_pass(mutant) else 3)
"""


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(tmp_path, name):
    old, new = MUTATIONS[name]
    so = _build_mutant(tmp_path, name, old, new)
    p = subprocess.run([sys.executable, "-c", _CHILD, ROOT, so], capture_output=True, text=True, timeout=300)
    assert p.returncode != 0, f"pins did not catch mutation {name}"
    assert p.returncode == 3 or p.returncode < 0, p.stderr[-2000:]
