"""Generator checks (no GPU): determinism and the structure each workload promises."""
from __future__ import annotations

import numpy as np
import pytest

import synth


def test_splitmix64_published_sequence():
    # SplitMix64 from state 0: the first outputs of the public reference code
    out = synth.splitmix64_sequence(0, 3)
    assert [int(x) for x in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_streams_are_deterministic_and_distinct():
    a = synth.Stream(3, 1, 2).u64(1000)
    b = synth.Stream(3, 1, 2).u64(1000)
    c = synth.Stream(3, 1, 3).u64(1000)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    st = synth.Stream(3, 1, 2)
    assert np.array_equal(np.concatenate([st.u64(400), st.u64(600)]), a)


def test_normal_moments():
    x = synth.Stream(1, 7).normal(200_000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_permutation_and_below():
    st = synth.Stream(8)
    p = st.permutation(5000)
    assert np.array_equal(np.sort(p), np.arange(5000))
    b = st.below(100_000, 7)
    assert b.min() == 0 and b.max() == 6


@pytest.mark.parametrize("i", [1, 2, 4])
def test_config_deterministic(i):
    assert synth.make_config(i).digest() == synth.make_config(i).digest()


def test_c1_structure():
    w = synth.make_config(1)
    assert w.scores.shape == (2, 8192) and w.k == 2048 and w.page_size == 64
    assert np.array_equal(np.sort(w.block_table[0]), np.arange(128))
    for r in range(2):
        # 409 copies of other positions: at least that many repeated values
        assert 8192 - np.unique(w.scores[r]).size >= 300


def test_c2_structure():
    w = synth.make_config(2)
    assert list(w.lengths) == [79_994 + r for r in range(7)]
    for r in range(7):
        n = w.lengths[r]
        row = w.scores[r]
        assert np.isneginf(row[n:]).all() and not np.isinf(row[:n]).any()
        frac0 = (row[:n] == 0).mean()
        assert 0.29 < frac0 < 0.31 and (row[:n] >= 0).all()
        assert not np.signbit(row[:n][row[:n] == 0]).any()     # +0.0 only


@pytest.mark.slow
def test_c3_structure():
    w = synth.make_config(3)
    assert w.scores.shape == (7, 1_000_000)
    lo, hi = np.float32(3.0), np.float32(3.0) + np.float32(2097 * 2.0 ** -22)
    for r in range(7):
        row = w.scores[r]
        inside = ((row >= lo) & (row <= hi)).sum()
        assert 10_000 <= inside <= 10_060       # the planted cluster plus rare normals
    assert np.array_equal(np.sort(w.block_table[0]), np.arange(15_625))


def test_c4_structure():
    w = synth.make_config(4)
    assert w.lengths.min() >= 512 and w.lengths.max() <= 200_000
    assert (w.lengths <= 2048).sum() >= 5
    assert w.bt_row_stride == 3125 and w.block_table.shape == (64, 3125)
    assert np.unique(w.block_table).size == 64 * 3125          # disjoint tables
    for r in range(64):
        assert np.isneginf(w.scores[r, w.lengths[r]:]).all()


def test_c5_structure():
    w = synth.make_config(5)
    s = w.scores
    assert all(np.unique(s[r]).size == 1 for r in range(0, 64, 9))
    assert all(np.unique(s[r]).size <= 16 for r in range(64, 128, 9))
    g2 = s[128:192]
    assert g2.min() >= 1.0 and g2.max() < 1.0 + 2.0 ** -12
    assert (g2.astype(np.float16) == np.float16(1.0)).all()     # one fp16 value
    assert all((np.diff(s[r]) <= 0).all() for r in range(192, 256, 9))
    assert np.unique(w.block_table).size == 256 * 2048


def test_random_case_junk_past_len():
    w = synth.random_case(5, rows=8, max_len=300, special=True)
    for r in range(8):
        assert (w.scores[r, w.lengths[r]:] == np.float32(1e30)).all()
