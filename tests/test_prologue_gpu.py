"""GPU parity of the fused indexer key prologue against the oracle
(oracle/prologue.py), through the C ABI.

Comparison rule (the FP8 codes are integers that FP32 arithmetic decides):
- slots: exact. Every slot the oracle writes holds the kernel's row; every
  other slot keeps its sentinel bytes (no stray stores).
- scales: relative difference at most 1e-5. The kernel's FP32 LayerNorm and
  rotation differ from the oracle's float64 ones by a few FP32 ulps of the
  token's largest value; 1e-5 is about 80 ulps, while a wrong formula (an
  unbiased variance, a missing bias, a lost rotation) moves the scale by far
  more.
- codes: equal, except where the oracle's scaled value lies within a relative
  1e-5 of the midpoint between two adjacent E4M3 values: there the two FP32
  computations may round to either neighbour, and the kernel's code must be
  one of the two. Such cases are rare (a bound on their count is checked).
- the kernel's own FP32 -> E4M3 conversion is bit-exact with the oracle's
  encoder on every code value, every tie and both neighbours of each, and
  random values (the quantizer's rounding, checked alone).
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import prologue as P
from tests import _gpu

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    HAVE_GPU = False

pytestmark = pytest.mark.gpu
if not HAVE_GPU:
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_indexer_amd import prologue as K  # noqa: E402

SENTINEL = 0xA5
SCALE_SENTINEL = -7.0


def run_kernel(w: synth.KeyPrologueInputs, with_status: bool = True, cos_sin_rows: int | None = None):
    dev = torch.device("cuda:0")
    k_act = torch.from_numpy(w.k_act.view(np.int16)).to(dev)
    cs = None
    if w.rope_dim:
        tab = w.cos_sin if cos_sin_rows is None else w.cos_sin[:cos_sin_rows]
        cs = torch.from_numpy(np.ascontiguousarray(tab)).to(dev)
    cache = torch.full((w.num_slots, 128), SENTINEL, dtype=torch.uint8, device=dev)
    scale = torch.full((w.num_slots,), SCALE_SENTINEL, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev) if with_status else None
    K.indexer_key_prologue(k_act, torch.from_numpy(w.weight).to(dev), torch.from_numpy(w.bias).to(dev), w.eps,
                           cs, w.rope_dim, torch.from_numpy(w.positions).to(dev),
                           torch.from_numpy(w.token_row).to(dev),
                           torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev), w.bt_row_stride,
                           w.page_size, cache, scale, status)
    torch.cuda.synchronize()
    return cache.cpu().numpy(), scale.cpu().numpy(), (int(status.item()) if with_status else 0)


def oracle_of(w: synth.KeyPrologueInputs):
    return P.key_prologue(w.k_act[:, :w.dim], w.weight, w.bias, w.eps, w.cos_sin, w.rope_dim, w.positions,
                          w.token_row, w.block_table, w.bt_row_stride, w.page_size)


def assert_codes_match(got: np.ndarray, want: np.ndarray, scaled: np.ndarray, label: str) -> int:
    """Codes equal, or adjacent with the oracle's value within 1e-5 of their midpoint."""
    diff = got != want
    n = int(diff.sum())
    if n == 0:
        return 0
    vg, vw = P.e4m3_decode(got[diff]), P.e4m3_decode(want[diff])
    x = np.clip(scaled[diff], -448.0, 448.0)
    mid = (vg + vw) / 2
    lo, hi = np.minimum(np.abs(vg), np.abs(vw)), np.maximum(np.abs(vg), np.abs(vw))
    pos = P._E4M3_POS
    # adjacent: no E4M3 magnitude strictly between them, same sign (or zero)
    between = np.searchsorted(pos, hi, side="left") - np.searchsorted(pos, lo, side="right")
    same_side = (np.sign(vg) == np.sign(vw)) | (vg == 0) | (vw == 0)
    near = np.abs(x - mid) <= 1e-5 * np.maximum(np.abs(x), 2.0 ** -9)
    ok = (between == 0) & same_side & near
    assert ok.all(), f"{label}: {int((~ok).sum())} codes differ beyond a rounding tie, e.g. " \
                     f"got {got[diff][~ok][:4]} want {want[diff][~ok][:4]} scaled {x[~ok][:4]}"
    assert n <= max(4, got.size // 1000), f"{label}: {n} codes at rounding ties"
    return n


def check(w: synth.KeyPrologueInputs, label: str) -> None:
    cache, scale, st = run_kernel(w)
    assert st == 0, f"{label}: device status {st:#x}"
    slots, codes, scales, pre, scaled = oracle_of(w)
    live = slots >= 0
    written = np.zeros(w.num_slots, bool)
    written[slots[live]] = True
    # untouched slots keep the sentinel
    assert (cache[~written] == SENTINEL).all() and (scale[~written] == SCALE_SENTINEL).all(), label
    got_codes = cache[slots[live]]
    assert_codes_match(got_codes, codes[live], scaled[live], label)
    rel = np.abs(scale[slots[live]].astype(np.float64) - scales[live]) / scales[live]
    assert rel.max(initial=0.0) <= 1e-5, f"{label}: scale rel err {rel.max():.3g}"


CASES = [
    dict(tokens=1),
    dict(tokens=17, rope_dim=128, page_size=16),
    dict(tokens=1000, rows=3),
    dict(tokens=100, rope_dim=0, shared_table=True, page_size=1),
    dict(tokens=333, rows=5, pad_every=5),
    dict(tokens=64, k_stride=136, rows=2),
    dict(tokens=4096, rows=7, page_size=64, act_scale=0.01),
    dict(tokens=2000, rows=2, act_scale=300.0, rope_dim=32),
]


@pytest.mark.parametrize("case", CASES, ids=[",".join(f"{k}={v}" for k, v in c.items()) for c in CASES])
def test_key_prologue_parity(case):
    w = synth.make_key_prologue(seed=40 + case["tokens"], **case)
    _gpu.say(f"[prologue] {case}")
    check(w, str(case))


def test_key_prologue_full_size():
    """The benchmarked batch: 131,072 tokens of 8 requests."""
    w = synth.make_key_prologue(131_072, seed=12, rows=8)
    _gpu.say("[prologue] full size 131072 tokens")
    check(w, "full size")


def test_key_prologue_zero_tokens_is_a_no_op():
    w = synth.make_key_prologue(0, seed=3)
    cache, scale, st = run_kernel(w)
    assert st == 0 and (cache == SENTINEL).all() and (scale == SCALE_SENTINEL).all()


def test_key_prologue_flags_bad_positions_and_slots():
    w = synth.make_key_prologue(200, seed=5, rows=2)
    w.positions = w.positions.copy()
    w.positions[7] = w.cos_sin.shape[0] + 3          # past the rotary table
    w.block_table = w.block_table.copy()
    r, p = int(w.token_row[150]), int(w.positions[150]) // w.page_size
    w.block_table[r, p] = w.num_slots // w.page_size + 9    # a page past the cache
    cache, scale, st = run_kernel(w)
    assert st & K.DEVICE_BAD_POSITION and st & K.DEVICE_BAD_SLOT
    # the other tokens are stored as usual
    w2 = synth.make_key_prologue(200, seed=5, rows=2)
    slots, codes, scales, _, scaled = oracle_of(w2)
    keep = np.ones(200, bool)
    keep[7] = False
    keep &= (w2.token_row != r) | (w2.positions // w2.page_size != p)
    assert_codes_match(cache[slots[keep]], codes[keep], scaled[keep], "flags")


def test_kernel_fp8_conversion_is_the_oracle_encoder():
    v = P.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2
    base = np.concatenate([v, mids]).astype(np.float32)
    st = synth.Stream(9, 1)
    x = np.concatenate([base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf)),
                        ((st.uniform(1_000_000) * 2 - 1) * 460.0).astype(np.float32),
                        ((st.uniform(100_000) * 2 - 1) * 2.0 ** -6).astype(np.float32),
                        np.array([449.0, 470.0, 1e6, 3e38, 0.0, -0.0], np.float32)]).astype(np.float32)
    x = np.concatenate([x, -x])
    got = K.debug_fp8(torch.from_numpy(x).to("cuda:0")).cpu().numpy()
    want = P.e4m3_encode(x.astype(np.float64))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} conversions differ, e.g. x={x[bad[:5]]} got {got[bad[:5]]} want {want[bad[:5]]}"
