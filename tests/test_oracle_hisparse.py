"""Pins for the HiSparse resolver oracle (no GPU): a hand-worked sequence of
four steps (resident reads, misses served in position order into empty then
least-recently-used slots, hits refreshing their stamp, an evicted token
missing again, a step with more misses than evictable slots), invariants on
random step sequences (map and tags consistent, every served row holds the
token's host copy, nothing used this step is evicted, victims never more
recent than survivors), and planted mistakes that must fail a pin."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import hisparse as HS


def _hand_setup():
    ps = 4
    table = np.array([7, -1, -1, 2], np.int32)          # pages 1, 2 live only on the host
    host_table = np.arange(4, dtype=np.int32)
    hot_rows = np.array([100, 101, 102], np.int64)
    kv = np.zeros((128, 8), np.uint8)
    host = np.repeat(np.arange(16, dtype=np.uint8)[:, None], 8, axis=1)   # host row h holds bytes h
    return ps, table, host_table, hot_rows, kv, host, HS.HotState.empty(3, 16)


def test_hand_worked_steps():
    ps, table, host_table, hot_rows, kv, host, st = _hand_setup()
    rows, f = HS.resolve(1, [5, 13, 9, 2], table, host_table, ps, hot_rows, st, kv, host)
    assert list(rows) == [100, 9, 101, 30] and f == 0
    assert list(st.tag) == [5, 9, -1] and list(st.stamp) == [1, 1, 0]
    assert (kv[100] == 5).all() and (kv[101] == 9).all()
    rows, f = HS.resolve(2, [9, 6, 4], table, host_table, ps, hot_rows, st, kv, host)
    assert list(rows) == [101, 100, 102] and f == 0
    assert list(st.tag) == [6, 9, 4] and list(st.stamp) == [2, 2, 2] and st.map[5] == -1
    assert (kv[100] == 6).all() and (kv[102] == 4).all()
    rows, f = HS.resolve(3, [5, 4, -1], table, host_table, ps, hot_rows, st, kv, host)
    assert list(rows) == [100, 102, -1] and f == 0
    assert list(st.tag) == [5, 9, 4] and list(st.stamp) == [3, 2, 3] and st.map[6] == -1
    rows, f = HS.resolve(4, [8, 10, 11, 5], table, host_table, ps, hot_rows, st, kv, host)
    assert list(rows) == [101, 102, -1, 100] and f == HS.HOT_FULL
    assert list(st.tag) == [5, 8, 10] and list(st.stamp) == [4, 4, 4]
    assert st.map[9] == -1 and st.map[4] == -1 and st.map[11] == -1


def _random_run(resolve, seed=3, steps=12, ctx=3000, ps=16, hot=64, k=24):
    st_ = synth.Stream(seed, 2)
    pages = ctx // ps
    table = np.where(st_.uniform(pages) < 0.6, -1, st_.permutation(pages)).astype(np.int32)
    host_table = st_.permutation(pages).astype(np.int32)
    hot_rows = (pages * ps + st_.permutation(hot * 2)[:hot]).astype(np.int64)
    kv = np.zeros((pages * ps + hot * 2, 4), np.uint8)
    host = (st_.u64(pages * ps * 4) & np.uint64(0xFF)).astype(np.uint8).reshape(pages * ps, 4)
    st = HS.HotState.empty(hot, ctx)
    out = []
    for step in range(1, steps + 1):
        # half the selection repeats recent positions (hits), half is new
        sel = st_.permutation(ctx)[:k]
        if out:
            prev = [p for p in out[-1][0] if p >= 0][: k // 2]
            sel[: len(prev)] = prev
            sel = np.unique(sel)[:k]
        before = st.copy()
        rows, f = resolve(step, sel, table, host_table, ps, hot_rows, st, kv, host)
        out.append((sel, rows, f, before, st.copy(), kv.copy()))
    return out, table, host_table, hot_rows, kv, host, ps


def test_random_sequences_keep_the_invariants():
    out, table, host_table, hot_rows, kv, host, ps = _random_run(HS.resolve)
    for step, (sel, rows, f, before, after, kv) in enumerate(out, 1):
        tagged = after.tag >= 0
        assert np.all(after.map[after.tag[tagged]] == np.flatnonzero(tagged))
        mapped = np.flatnonzero(after.map >= 0)
        assert np.all(after.tag[after.map[mapped]] == mapped)
        for p, r in zip(sel, rows):
            page = table[p // ps]
            if page >= 0:
                assert r == page * ps + p % ps
            elif r >= 0:
                assert after.map[p] >= 0 and hot_rows[after.map[p]] == r and after.stamp[after.map[p]] == step
                assert (kv[r] == host[host_table[p // ps] * ps + p % ps]).all()
        evicted = [s for s in range(len(after.tag)) if before.tag[s] >= 0 and before.tag[s] != after.tag[s]]
        kept = [s for s in range(len(after.tag)) if after.stamp[s] != step]
        for s in evicted:
            assert before.stamp[s] != step
            assert all((before.stamp[s], s) < (after.stamp[u], u) for u in kept)


def _variant(sort_misses=True, lru=True, host_shift=0, refresh_hits=True):
    """The resolver with one rule changed (for the planted mistakes)."""
    def resolve(step, sel, table, host_table, ps, hot_rows, st, kv, host):
        sel = np.asarray(sel, np.int64)
        rows = np.full(sel.shape, -1, np.int64)
        misses = []
        for j, p in enumerate(sel):
            if p < 0:
                continue
            page = int(table[p // ps])
            if page >= 0:
                rows[j] = page * ps + p % ps
            elif st.map[p] >= 0:
                s = int(st.map[p])
                if refresh_hits:
                    st.stamp[s] = step
                rows[j] = int(hot_rows[s])
            else:
                misses.append((int(p), j))
        if sort_misses:
            misses.sort()
        cand = sorted((s for s in range(len(st.tag)) if int(st.stamp[s]) != step),
                      key=lambda s: (int(st.stamp[s]), s), reverse=not lru)
        flags = 0
        for i, (p, j) in enumerate(misses):
            if i >= len(cand):
                flags |= HS.HOT_FULL
                continue
            s = cand[i]
            if st.tag[s] >= 0:
                st.map[st.tag[s]] = -1
            st.tag[s], st.map[p], st.stamp[s] = p, s, step
            kv[int(hot_rows[s])] = host[(int(host_table[p // ps]) * ps + p % ps + host_shift) % len(host)]
            rows[j] = int(hot_rows[s])
        return rows, flags
    return resolve


def _pins_pass() -> bool:
    try:
        test_hand_worked_steps()
        test_random_sequences_keep_the_invariants()
    except (AssertionError, IndexError, KeyError):
        return False
    return True


MISTAKES = {"most_recent_victim": dict(lru=False), "misses_in_selection_order": dict(sort_misses=False),
            "wrong_host_row": dict(host_shift=1), "hits_not_refreshed": dict(refresh_hits=False)}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_hisparse_mistakes(monkeypatch, name):
    monkeypatch.setattr(HS, "resolve", _variant(**MISTAKES[name]))
    assert not _pins_pass()


def test_variant_without_changes_passes():
    """(the mutants' common code is the rule as stated)"""
    import oracle.hisparse as mod
    real = mod.resolve
    try:
        mod.resolve = _variant()
        assert _pins_pass()
    finally:
        mod.resolve = real


def test_pins_accept_real_hisparse_oracle():
    assert _pins_pass()
