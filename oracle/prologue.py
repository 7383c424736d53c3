"""CPU oracle for the indexer key prologue: LayerNorm, rotary embedding, FP8
quantization and the paged indexer-cache store of each new key token.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path. It shares
no code with the HIP library.

Source: the lmsys.org page "Serving GLM5.2 NVFP4 Agentic Workload with SGLang",
section "Indexer Prologue Fusion" (and its Figure 5). The page lists the fused
key path as LayerNorm, RoPE, FP8 quantization and the paged indexer KV-cache
store, fed by the key half of the fused BF16 projection, and says the fused
path quantizes the untransformed activations (no Hadamard transform). It gives
no formula for any step, so each step below is the textbook definition, and
every choice the page leaves open is a stated reading:

1. LayerNorm over the head dimension D (= 128): mean and biased variance,
   ``(x - mean) / sqrt(var + eps) * weight + bias``.
2. Rotary embedding (Su et al., "RoFormer", 2021) on the first ``rope_dim``
   dimensions, as interleaved pairs (2i, 2i+1) rotated by the angle of pair i
   at the token's position; the cosines and sines come from the caller's table
   ``cos_sin[pos] = [cos of pairs 0..R/2-1, sin of pairs 0..R/2-1]`` (the
   serving engines' rotary cache), so the oracle and the kernel read the same
   FP32 values and never evaluate a transcendental function.
3. FP8 E4M3 (OCP "fn" variant: bias 7, 3 mantissa bits, largest finite 448,
   no infinities) with one FP32 scale per token: ``scale = amax / 448`` with
   ``amax`` the largest |value| of the token after steps 1-2, floored at 2^-64
   so that ``448 / amax`` stays finite (an all-zero token stores zero codes),
   codes = round-to-nearest-even of ``value * (448 / amax)``, saturated at
   +-448.
4. Store: the token's physical slot is ``block_table[row][pos // page_size] *
   page_size + pos % page_size`` (the same slot formula as the top-k output);
   ``cache_fp8[slot] = codes`` (D bytes) and ``cache_scale[slot] = scale``.
   Tokens whose row index is negative are padding and store nothing.

Steps 1-2 are computed here in float64 and rounded once to float32. The
quantization (step 3) decides integers, so it runs in the kernel's precision:
FP32 ``amax``, FP32 ``448 / amax`` and FP32 products, exactly as stated above.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
AMAX_FLOOR = 2.0 ** -64


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) to float64: the top half of an FP32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3 (fn) codes to float64: sign, 4-bit exponent (bias 7), 3-bit
    mantissa; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# All 127 non-negative finite E4M3 values in increasing order (code = index).
_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of finite float values to E4M3 (fn) codes,
    saturating at +-448. The sign of zero is kept (-0 -> 0x80).

    Written from the format's value set: the nearest representable magnitude
    wins; on an exact tie the one with the even code (mantissa LSB 0) wins.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: finite inputs only")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")        # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    vhi, vlo = _E4M3_POS[hi], _E4M3_POS[lo]
    dlo, dhi = a - vlo, vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == vhi, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def layer_norm(x: np.ndarray, weight: np.ndarray, bias: np.ndarray, eps: float) -> np.ndarray:
    """Step 1 in float64 over the last axis (biased variance)."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * np.asarray(weight, np.float64) + np.asarray(bias, np.float64)


def rope_interleaved(y: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Step 2: rotate pairs (2i, 2i+1) of the first 2 * cos.shape[-1] dims:
    (a, b) -> (a cos - b sin, a sin + b cos). cos/sin are per token, [T, R/2]."""
    y = np.array(y, dtype=np.float64, copy=True)
    r2 = cos.shape[-1]
    a = y[..., 0:2 * r2:2].copy()
    b = y[..., 1:2 * r2:2].copy()
    c = np.asarray(cos, np.float64)
    s = np.asarray(sin, np.float64)
    y[..., 0:2 * r2:2] = a * c - b * s
    y[..., 1:2 * r2:2] = a * s + b * c
    return y


def quantize_fp32(v32: np.ndarray):
    """Step 3 on FP32 tokens [T, D]: (codes uint8 [T, D], scale float32 [T],
    scaled float64 [T, D] = the exact product before rounding to E4M3)."""
    v32 = np.asarray(v32, dtype=np.float32)
    amax = np.abs(v32).max(axis=-1)
    amax = np.maximum(amax, np.float32(AMAX_FLOOR)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / amax).astype(np.float32)          # FP32 division
    scaled32 = (v32 * inv[:, None]).astype(np.float32)             # FP32 products
    codes = e4m3_encode(scaled32.astype(np.float64))
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes, scale, scaled32.astype(np.float64)


def slots_of(positions, token_row, block_table, bt_row_stride: int, page_size: int) -> np.ndarray:
    """Step 4's slot per token (int64; -1 for padding tokens, row < 0)."""
    pos = np.asarray(positions, dtype=np.int64)
    row = np.zeros_like(pos) if token_row is None else np.asarray(token_row, dtype=np.int64)
    table = np.asarray(block_table, dtype=np.int64).reshape(-1)
    out = np.full(pos.shape, -1, np.int64)
    ok = row >= 0
    page = table[row[ok] * int(bt_row_stride) + pos[ok] // page_size]
    out[ok] = page * page_size + pos[ok] % page_size
    return out


def key_prologue(k_act_bf16, weight, bias, eps, cos_sin, rope_dim, positions, token_row,
                 block_table, bt_row_stride, page_size):
    """The whole key path for T tokens.

    Returns (slots int64 [T], codes uint8 [T, D], scales float32 [T],
    prequant float32 [T, D], scaled float64 [T, D]): the cache rows each token
    writes, and the intermediate values the parity tests use to place rounding
    boundaries."""
    x = bf16_to_f64(k_act_bf16)
    T, D = x.shape
    y = layer_norm(x, weight, bias, eps)
    if rope_dim:
        pos = np.asarray(positions, dtype=np.int64)
        tab = np.asarray(cos_sin, dtype=np.float32).reshape(-1, rope_dim)
        cos = tab[pos, : rope_dim // 2].astype(np.float64)
        sin = tab[pos, rope_dim // 2:].astype(np.float64)
        y = rope_interleaved(y, cos, sin)
    pre = y.astype(np.float32)
    codes, scales, scaled = quantize_fp32(pre)
    slots = slots_of(positions, token_row, block_table, bt_row_stride, page_size)
    return slots, codes, scales, pre, scaled


def store(cache_fp8: np.ndarray, cache_scale: np.ndarray, slots, codes, scales) -> None:
    """Apply step 4 to host copies of the cache (padding tokens skipped)."""
    for t, s in enumerate(np.asarray(slots)):
        if s >= 0:
            cache_fp8[s] = codes[t]
            cache_scale[s] = scales[t]
