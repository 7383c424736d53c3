"""Pins for the indexer score oracle (no GPU): the MQA logits against an
independent loop implementation and closed forms (one-hot queries, the ReLU
identity, linearity in the gate weights, paging invariance), and the query
prologue's head-gate folding against the unquantized score within the FP8
error. Planted mistakes must fail a pin."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import indexer_logits as L
from oracle import prologue as P


def _case(seed=1, T=2, H=3, D=8, n=40, ps=4):
    st = synth.Stream(seed, 5)
    q = P.e4m3_encode(st.normal(T * H * D).reshape(T, H, D) * 30)
    pages = (n + ps - 1) // ps
    table = st.permutation(pages + 2)[:pages][None, :].astype(np.int32)
    slots = (pages + 2) * ps
    k = P.e4m3_encode(st.normal(slots * D).reshape(slots, D) * 30)
    ks = (0.01 + st.uniform(slots)).astype(np.float32)
    w = (st.normal(T * H).reshape(T, H)).astype(np.float32)
    lengths = np.array([n, n // 2 + 1][:T] + [n] * max(0, T - 2), np.int64)
    return q, w, k, ks, table, ps, lengths


def test_logits_match_loop_implementation():
    q, w, k, ks, table, ps, lengths = _case()
    got = L.mqa_logits(q, w, k, ks, table, 0, ps, lengths)
    ref = L.mqa_logits_loops(q, w, k, ks, table, 0, ps, lengths)
    for (t, s), v in ref.items():
        assert abs(got[t, s] - v) <= 1e-12 * max(1.0, abs(v)), (t, s)
    assert np.isnan(got[1, int(lengths[1]):]).all()


def test_logits_one_hot_query():
    _, _, k, ks, table, ps, _ = _case(D=8)
    q = np.zeros((1, 1, 8), np.uint8)
    q[0, 0, 5] = 0x38                                          # 1.0 on dim 5
    got = L.mqa_logits(q, np.ones((1, 1), np.float32), k, ks, table, 0, ps, [12])
    slots = P.slots_of(np.arange(12), None, table, 0, ps)
    want = ks[slots] * np.maximum(P.e4m3_decode(k[slots, 5]), 0.0)
    assert np.allclose(got[0], want, rtol=1e-15, atol=0)


def test_logits_relu_identity_and_linearity():
    q, w, k, ks, table, ps, lengths = _case(H=1)
    a = L.mqa_logits(q, w, k, ks, table, 0, ps, lengths)
    b = L.mqa_logits(q ^ np.uint8(0x80), w, k, ks, table, 0, ps, lengths)   # every q negated
    one = np.ones_like(w)
    dots = L.mqa_logits(q, one, k, ks, table, 0, ps, lengths) - L.mqa_logits(q ^ np.uint8(0x80), one, k, ks,
                                                                                table, 0, ps, lengths)
    # ReLU(x) + ReLU(-x) = |x|; ReLU(x) - ReLU(-x) = x
    assert np.allclose(a + b, w[:, :1] * np.abs(dots), equal_nan=True)
    assert np.allclose(L.mqa_logits(q, 2 * w, k, ks, table, 0, ps, lengths), 2 * a, equal_nan=True)


def test_logits_paging_invariance():
    q, w, k, ks, table, ps, lengths = _case()
    a = L.mqa_logits(q, w, k, ks, table, 0, ps, lengths)
    # the same keys in an identity-paged cache
    slots = P.slots_of(np.arange(int(lengths.max())), None, table, 0, ps)
    k2, ks2 = k[slots], ks[slots]
    ident = np.arange((len(slots) + ps - 1) // ps, dtype=np.int32)[None, :]
    b = L.mqa_logits(q, w, k2, ks2, ident, 0, ps, lengths)
    assert np.array_equal(np.nan_to_num(a, nan=-1), np.nan_to_num(b, nan=-1))


def test_query_prologue_folds_scales_into_the_gate():
    st = synth.Stream(3, 9)
    T, H, D = 3, 4, 128
    qraw = st.normal(T * H * D).reshape(T, H, D) * 2
    bits = synth.bf16_bits(qraw)
    w_raw = st.normal(T * H).reshape(T, H).astype(np.float32)
    cs = synth.rotary_table(64, 64)
    pos = np.array([3, 17, 60])
    codes, wq, _ = L.query_prologue(bits, w_raw, 0.125, cs, 64, pos)
    # unquantized reference: the same rotary (already pinned) on the BF16 values
    qf = P.bf16_to_f64(bits)
    cos = np.repeat(cs[pos, :32].astype(np.float64)[:, None, :], H, 1)
    sin = np.repeat(cs[pos, 32:].astype(np.float64)[:, None, :], H, 1)
    qf = P.rope_interleaved(qf, cos, sin)
    keys = st.normal(50 * D).reshape(50, D)
    ref = 0.125 * np.einsum("th,ths->ts", w_raw.astype(np.float64),
                            np.maximum(np.einsum("thd,sd->ths", qf, keys), 0))
    got = np.einsum("th,ths->ts", wq.astype(np.float64),
                    np.maximum(np.einsum("thd,sd->ths", P.e4m3_decode(codes), keys), 0))
    # FP8 keeps ~4 significant bits: the dot products agree to a few percent
    # of their magnitude sums
    mag = 0.125 * np.einsum("th,ths->ts", np.abs(w_raw).astype(np.float64),
                            np.einsum("thd,sd->ths", np.abs(qf), np.abs(keys)))
    assert np.all(np.abs(got - ref) <= 0.07 * mag)
    # and each head's amax element is +-448
    am = np.abs(P.bf16_to_f64(bits)).max(axis=-1)
    assert ((codes == 0x7E) | (codes == 0xFE)).any(axis=-1).all()


_ORIG = L.mqa_logits


def _relu_after_sum(q_codes, w, kc, ks, table, stride, ps, lengths, token_row=None, positions_of=None):
    T, H, D = q_codes.shape
    out = np.full((T, int(max(lengths))), np.nan)
    qd = P.e4m3_decode(q_codes)
    for t in range(T):
        n = int(lengths[t])
        slots = P.slots_of(np.arange(n), None, table, stride, ps)
        out[t, :n] = ks[slots] * np.maximum(np.asarray(w[t], np.float64) @ (qd[t] @ P.e4m3_decode(kc[slots]).T), 0)
    return out


def _no_relu(q_codes, w, kc, ks, table, stride, ps, lengths, token_row=None, positions_of=None):
    T, H, D = q_codes.shape
    out = np.full((T, int(max(lengths))), np.nan)
    qd = P.e4m3_decode(q_codes)
    for t in range(T):
        n = int(lengths[t])
        slots = P.slots_of(np.arange(n), None, table, stride, ps)
        out[t, :n] = ks[slots] * (np.asarray(w[t], np.float64) @ (qd[t] @ P.e4m3_decode(kc[slots]).T))
    return out


def _k_scale_dropped(q_codes, w, kc, ks, *args, **kw):
    return _ORIG(q_codes, w, kc, np.ones_like(ks), *args, **kw)


def _slot_unpaged(q_codes, w, kc, ks, table, stride, ps, lengths, token_row=None, positions_of=None):
    ident = np.arange(kc.shape[0] // ps, dtype=np.int32)[None, :]
    return _ORIG(q_codes, w, kc, ks, ident, 0, ps, lengths)


def _pins_pass() -> bool:
    try:
        test_logits_match_loop_implementation()
        test_logits_one_hot_query()
        test_logits_relu_identity_and_linearity()
        test_logits_paging_invariance()
    except (AssertionError, ValueError, IndexError):
        return False
    return True


@pytest.mark.parametrize("fn", [_relu_after_sum, _no_relu, _k_scale_dropped, _slot_unpaged],
                         ids=lambda f: f.__name__.strip("_"))
def test_planted_logits_mistakes(monkeypatch, fn):
    monkeypatch.setattr(L, "mqa_logits", fn)
    assert not _pins_pass()


def test_pins_accept_real_logits_oracle():
    assert _pins_pass()


def test_logits_at_positions_is_the_row_restricted():
    q, w, k, ks, table, ps, lengths = _case(T=2)
    full = L.mqa_logits(q, w, k, ks, table, 0, ps, lengths)
    bound = L.error_bound(q, w, k, ks, table, 0, ps, lengths)
    pos = np.array([0, 3, 17, int(lengths[1]) - 1])
    for t in range(2):
        s, b = L.mqa_logits_at(q, w, k, ks, table, 0, ps, t, pos)
        assert np.allclose(s, full[t, pos], rtol=1e-14) and np.allclose(b, bound[t, pos], rtol=1e-14)
