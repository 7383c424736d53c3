"""Pins for the key-prologue oracle (no GPU).

Each step is checked against something other than itself: the E4M3 encoder
against torch's own float8_e4m3fn conversion and against hand-decoded codes;
LayerNorm against torch.nn.functional.layer_norm in float64 and closed forms;
the rotary step against its defining properties (pair norms kept, angle zero
is the identity, a quarter turn, and dot products that depend only on the
position difference); the quantizer against its error bound and the amax
element; the slots against the identity table and a hand-worked case; and the
whole path against a hand-worked token. Planted mistakes in each step must
fail a pin.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import prologue as P


# --- E4M3 --------------------------------------------------------------------

def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_decode_hand_values():
    assert P.e4m3_decode(np.array([0x7E]))[0] == 448.0          # largest finite
    assert P.e4m3_decode(np.array([0x38]))[0] == 1.0            # exponent 7, mantissa 0
    assert P.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6      # smallest normal
    assert P.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9      # smallest subnormal
    assert P.e4m3_decode(np.array([0x07]))[0] == 7 * 2.0 ** -9  # largest subnormal
    assert P.e4m3_decode(np.array([0xBC]))[0] == -1.5           # sign, mantissa 4/8
    assert np.isnan(P.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    v = P.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)                                # codes 0..126 increase


def _boundary_cases() -> np.ndarray:
    v = P.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2                                  # exact ties
    f32 = np.concatenate([v, mids]).astype(np.float32)
    up = np.nextafter(f32, np.float32(np.inf))
    dn = np.nextafter(f32, np.float32(-np.inf))
    st = synth.Stream(5, 77)
    rnd = (st.uniform(200_000) * 2 - 1) * 448.0
    tiny = (st.uniform(20_000) * 2 - 1) * 2.0 ** -5
    x = np.concatenate([f32, up, dn, rnd, tiny]).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    return np.concatenate([x, -x])


def test_e4m3_encode_matches_torch_conversion():
    x = _boundary_cases()
    assert np.array_equal(P.e4m3_encode(x.astype(np.float64)), _torch_e4m3(x))


def test_e4m3_encode_saturates_and_keeps_zero_sign():
    big = np.array([448.0, 449.0, 463.99, 464.0, 1e6, 3.0e38])
    assert list(P.e4m3_encode(big)) == [0x7E] * 6
    assert list(P.e4m3_encode(-big)) == [0xFE] * 6
    assert list(P.e4m3_encode(np.array([0.0, -0.0]))) == [0x00, 0x80]


# --- LayerNorm ---------------------------------------------------------------

def test_layer_norm_matches_torch_float64():
    st = synth.Stream(6, 1)
    x = st.normal(50 * 128).reshape(50, 128) * 4 + 1.5
    w, b = st.normal(128), st.normal(128)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), torch.from_numpy(w),
                                         torch.from_numpy(b), eps=1e-6).numpy()
    assert np.allclose(P.layer_norm(x, w, b, 1e-6), ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_closed_forms():
    w, b = np.linspace(0.5, 2, 128), np.linspace(-1, 1, 128)
    assert np.allclose(P.layer_norm(np.full((2, 128), 7.25), w, b, 1e-6), b)     # constant row -> bias
    alt = np.tile([3.0, -3.0], 64)[None, :]                                       # mean 0, var 9
    assert np.allclose(P.layer_norm(alt, np.ones(128), np.zeros(128), 0.0), alt / 3.0)
    x = synth.Stream(6, 2).normal(128)[None, :]
    assert np.allclose(P.layer_norm(x + 100.0, w, b, 1e-6), P.layer_norm(x, w, b, 1e-6), atol=1e-9)


# --- rotary embedding ------------------------------------------------------

def _table64(max_pos: int, rope_dim: int) -> tuple[np.ndarray, np.ndarray]:
    inv = 10000.0 ** (-np.arange(0, rope_dim, 2) / rope_dim)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def test_rope_keeps_pair_norms_and_rest():
    st = synth.Stream(6, 3)
    y = st.normal(20 * 128).reshape(20, 128)
    cos, sin = _table64(20, 64)
    r = P.rope_interleaved(y, cos, sin)
    n0 = y[:, 0:64:2] ** 2 + y[:, 1:64:2] ** 2
    n1 = r[:, 0:64:2] ** 2 + r[:, 1:64:2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)
    assert np.array_equal(r[:, 64:], y[:, 64:])                 # dims past rope_dim untouched
    assert np.allclose(r[0], y[0])                               # position 0: angle 0


def test_rope_quarter_turn():
    y = np.zeros((1, 4))
    y[0, 0] = 1.0                                                # pair 0 = (1, 0)
    r = P.rope_interleaved(y, np.array([[0.0]]), np.array([[1.0]]))
    assert np.allclose(r[0], [0.0, 1.0, 0.0, 0.0])


def test_rope_dot_products_depend_on_position_difference():
    st = synth.Stream(6, 4)
    q, k = st.normal(128), st.normal(128)
    cos, sin = _table64(400, 128)

    def dot(m, n):
        a = P.rope_interleaved(q[None, :], cos[m:m + 1], sin[m:m + 1])
        b = P.rope_interleaved(k[None, :], cos[n:n + 1], sin[n:n + 1])
        return float((a @ b.T).item())

    for m, n, d in [(5, 3, 100), (0, 7, 250), (30, 30, 1)]:
        assert abs(dot(m, n) - dot(m + d, n + d)) < 1e-9
    assert abs(dot(9, 2) - dot(2, 9)) > 1e-3                     # and not symmetric in it


# --- quantizer and slots -----------------------------------------------------

def test_quantize_amax_code_and_error_bound():
    st = synth.Stream(6, 5)
    v = (st.normal(40 * 128).reshape(40, 128) * np.exp(st.normal(40))[:, None]).astype(np.float32)
    codes, scale, scaled = P.quantize_fp32(v)
    am = np.abs(v).argmax(axis=1)
    top = codes[np.arange(40), am]
    assert np.all((top == 0x7E) | (top == 0xFE))                 # the amax element is +-448
    deq = P.e4m3_decode(codes) * scale[:, None].astype(np.float64)
    # RNE error: half the spacing of E4M3 at the value (2^(e-3) / 2 in the
    # binade 2^e; 2^-10 for subnormals), in scaled units
    a = np.abs(scaled)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half = np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
    err = np.abs(deq - v.astype(np.float64)) / scale[:, None]
    assert np.all(err <= half * (1 + 1e-6) + 448 * 2.0 ** -23)


def test_quantize_zero_token():
    codes, scale, _ = P.quantize_fp32(np.zeros((1, 128), np.float32))
    assert not codes.any() and scale[0] == np.float32(2.0 ** -64) / np.float32(448.0)


def test_slots_identity_and_hand_case():
    pos = np.arange(300)
    assert np.array_equal(P.slots_of(pos, None, np.arange(5)[None, :], 0, 64), pos)
    bt = np.array([[4, 1, 7], [2, 0, 5]])
    s = P.slots_of(np.array([0, 63, 64, 130, 5, 70]), np.array([0, 0, 0, 0, 1, -1]), bt, 3, 64)
    assert list(s) == [256, 319, 64, 450, 133, -1]


def test_whole_token_hand_worked():
    # alternating +a/-a: LayerNorm gives +-1 (eps 0, weight 1, bias 0); angle 0
    # leaves it; amax 1 -> codes +-448, scale 1/448
    a = 1.5
    x = np.tile([a, -a], 64).astype(np.float64)
    bits = synth.bf16_bits(x)[None, :]
    cs = synth.rotary_table(1, 64)
    slots, codes, scales, pre, _ = P.key_prologue(bits, np.ones(128), np.zeros(128), 0.0, cs, 64,
                                                  np.array([0]), None, np.array([[9]]), 0, 16)
    assert slots[0] == 9 * 16
    assert list(codes[0, :4]) == [0x7E, 0xFE, 0x7E, 0xFE]
    assert scales[0] == np.float32(1.0) / np.float32(448.0)


# --- planted mistakes --------------------------------------------------------

def _pins_pass() -> bool:
    tests = [test_e4m3_decode_hand_values, test_e4m3_encode_matches_torch_conversion,
             test_e4m3_encode_saturates_and_keeps_zero_sign, test_layer_norm_matches_torch_float64,
             test_layer_norm_closed_forms, test_rope_keeps_pair_norms_and_rest, test_rope_quarter_turn,
             test_rope_dot_products_depend_on_position_difference, test_quantize_amax_code_and_error_bound,
             test_quantize_zero_token, test_slots_identity_and_hand_case, test_whole_token_hand_worked]
    try:
        for t in tests:
            t()
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def _ln_unbiased(x, weight, bias, eps):
    x = np.asarray(x, np.float64)
    m = x.mean(axis=-1, keepdims=True)
    v = ((x - m) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - m) / np.sqrt(v + eps) * weight + bias


_ORIG_ROPE = P.rope_interleaved
_ORIG_SLOTS = P.slots_of


def _rope_sign_flip(y, cos, sin):
    return _ORIG_ROPE(y, cos, -np.asarray(sin))


def _rope_half_split(y, cos, sin):
    y = np.array(y, np.float64, copy=True)
    r2 = cos.shape[-1]
    a, b = y[..., :r2].copy(), y[..., r2:2 * r2].copy()
    y[..., :r2] = a * cos - b * sin
    y[..., r2:2 * r2] = a * sin + b * cos
    return y


def _encode_truncating(x):
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    code = (np.searchsorted(P._E4M3_POS, a, side="right") - 1).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def _encode_ties_away(x):
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.minimum(np.searchsorted(P._E4M3_POS, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    pick = (P._E4M3_POS[hi] - a) <= (a - P._E4M3_POS[lo])
    code = np.where(pick, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def _slots_offset_dropped(positions, token_row, block_table, bt_row_stride, page_size):
    s = _ORIG_SLOTS(positions, token_row, block_table, bt_row_stride, page_size)
    pos = np.asarray(positions, np.int64)
    return np.where(s >= 0, s - pos % page_size, s)


MISTAKES = {
    "layer_norm_unbiased_variance": ("layer_norm", _ln_unbiased),
    "rope_sine_sign": ("rope_interleaved", _rope_sign_flip),
    "rope_half_split_pairs": ("rope_interleaved", _rope_half_split),
    "e4m3_truncates": ("e4m3_encode", _encode_truncating),
    "e4m3_ties_away": ("e4m3_encode", _encode_ties_away),
    "slot_offset_dropped": ("slots_of", _slots_offset_dropped),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_prologue_mistakes(monkeypatch, name):
    attr, fn = MISTAKES[name]
    monkeypatch.setattr(P, attr, fn)
    assert not _pins_pass(), f"pins did not catch {name}"


def test_pins_accept_real_prologue_oracle():
    assert _pins_pass()
