"""CPU oracle for the indexer's score producer: the query prologue (rotary,
FP8 E4M3 quantization, head-gate scaling) and the MQA logits over the paged
FP8 key cache, whose rows the top-k selects from.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path. It shares
no code with the HIP library.

Sources: the lmsys.org page "Serving GLM5.2 NVFP4 Agentic Workload with
SGLang". Section "Kernel Optimization / TopK-V2" says the DSA indexer turns
each query into scores over historical KV positions; section "Indexer
Prologue Fusion" lists the query path as RoPE, FP8 quantization and
head-gate scaling (the raw head-gate weights come from the fused
wk_weights_proj projection), and the key path stores FP8 keys in the paged
indexer cache; section "What's Next" names the MQA logits kernel. The page
prints no formula. The reading implemented here is the lightning indexer's
published score (DeepSeek-V3.2 technical report): for query token t with
H indexer heads and a key at position s,

    score[t][s] = sum_h  w[t][h] * ReLU( q[t][h] . k[s] ),

evaluated on the quantized operands, with every scale that commutes with
the ReLU folded outside it (all scales are positive):

    q[t][h] = decode(q_codes[t][h]) * q_scale[t][h]
    k[s]    = decode(k_codes[slot(s)]) * k_scale[slot(s)]
    w'[t][h] = w_raw[t][h] * q_scale[t][h] * gate_scale    (head-gate scaling)
    score[t][s] = k_scale[slot(s)] * sum_h w'[t][h] * ReLU(decode(q_codes[t][h]) . decode(k_codes[slot(s)]))

`gate_scale` is the caller's constant (the serving engines use
H^-1/2 * D^-1/2). The query quantizer is the key path's (per token and head:
scale = amax / 448, codes = RNE of value * 448 / amax in FP32). Scores are
produced for s in [0, lengths[t]) (causal verify/prefill rows); the slot of
position s is the top-k library's block-table formula.
"""
from __future__ import annotations

import numpy as np

from oracle import prologue as P


def query_prologue(q_bf16: np.ndarray, w_raw: np.ndarray, gate_scale: float, cos_sin, rope_dim: int,
                   positions):
    """q_bf16: uint16 [T, H, D] BF16 bits; w_raw: float32 [T, H].

    Returns (codes uint8 [T, H, D], w' float32 [T, H], scaled float64 [T, H, D]
    = each code's exact FP32 input, for placing rounding ties). Rotary and the
    FP32 rounding as in the key path; w' = fp32(fp32(w_raw * q_scale) * gate_scale)."""
    q = P.bf16_to_f64(q_bf16)
    T, H, D = q.shape
    if rope_dim:
        pos = np.asarray(positions, dtype=np.int64)
        tab = np.asarray(cos_sin, dtype=np.float32).reshape(-1, rope_dim)
        cos = np.repeat(tab[pos, : rope_dim // 2].astype(np.float64)[:, None, :], H, axis=1)
        sin = np.repeat(tab[pos, rope_dim // 2:].astype(np.float64)[:, None, :], H, axis=1)
        q = P.rope_interleaved(q, cos, sin)
    pre = q.astype(np.float32).reshape(T * H, D)
    codes, scale, scaled = P.quantize_fp32(pre)
    w = (np.asarray(w_raw, np.float32).reshape(T * H) * scale).astype(np.float32)
    w = (w * np.float32(gate_scale)).astype(np.float32)
    return codes.reshape(T, H, D), w.reshape(T, H), scaled.reshape(T, H, D)


def mqa_logits(q_codes: np.ndarray, w: np.ndarray, k_cache_fp8: np.ndarray, k_cache_scale: np.ndarray,
               block_table, bt_row_stride: int, page_size: int, lengths, token_row=None,
               positions_of=None) -> np.ndarray:
    """Scores float64 [T, max(lengths)] (NaN past each row's length).

    q_codes uint8 [T, H, D]; w float32 [T, H] (the head-gate weights after
    scaling); the key cache as the key path stores it. Row t reads the keys at
    positions [0, lengths[t]) of request token_row[t] (all request 0 when
    token_row is None)."""
    T, H, D = q_codes.shape
    lengths = np.asarray(lengths, dtype=np.int64)
    L = int(lengths.max()) if T else 0
    out = np.full((T, L), np.nan)
    qd = P.e4m3_decode(q_codes)                         # [T, H, D]
    for t in range(T):
        n = int(lengths[t])
        if n == 0:
            continue
        row = 0 if token_row is None else int(token_row[t])
        s = np.arange(n, dtype=np.int64)
        slots = P.slots_of(s, np.full(n, row), block_table, bt_row_stride, page_size)
        kd = P.e4m3_decode(k_cache_fp8[slots])          # [n, D]
        dots = qd[t] @ kd.T                             # [H, n], exact products and sums in float64
        out[t, :n] = k_cache_scale[slots].astype(np.float64) * (np.asarray(w[t], np.float64) @ np.maximum(dots, 0.0))
    return out


def mqa_logits_loops(q_codes, w, k_cache_fp8, k_cache_scale, block_table, bt_row_stride, page_size, lengths):
    """The same scores by plain Python loops over tokens, positions, heads
    and dims (tiny inputs, one block-table row shared by every token):
    score = k_scale * sum_h w * max(0, sum_d q*k)."""
    T, H, D = q_codes.shape
    table = np.asarray(block_table).reshape(-1)
    out = {}
    for t in range(T):
        for s in range(int(lengths[t])):
            slot = int(table[s // page_size]) * page_size + s % page_size
            acc = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += float(P.e4m3_decode(np.array([q_codes[t, h, d]]))[0]) * \
                        float(P.e4m3_decode(np.array([k_cache_fp8[slot, d]]))[0])
                acc += float(w[t, h]) * max(0.0, dot)
            out[(t, s)] = float(k_cache_scale[slot]) * acc
    return out


def error_bound(q_codes, w, k_cache_fp8, k_cache_scale, block_table, bt_row_stride, page_size, lengths,
                token_row=None):
    """Per score, the magnitude sum the FP32 evaluation's rounding scales with:
    k_scale * sum_h |w| * sum_d |q * k| (float64 [T, L], NaN past the length)."""
    T, H, D = q_codes.shape
    lengths = np.asarray(lengths, dtype=np.int64)
    L = int(lengths.max()) if T else 0
    out = np.full((T, L), np.nan)
    qa = np.abs(P.e4m3_decode(q_codes))
    for t in range(T):
        n = int(lengths[t])
        if n == 0:
            continue
        row = 0 if token_row is None else int(token_row[t])
        slots = P.slots_of(np.arange(n), np.full(n, row), block_table, bt_row_stride, page_size)
        ka = np.abs(P.e4m3_decode(k_cache_fp8[slots]))
        out[t, :n] = k_cache_scale[slots] * (np.abs(np.asarray(w[t], np.float64)) @ (qa[t] @ ka.T))
    return out


def mqa_logits_at(q_codes, w, k_cache_fp8, k_cache_scale, block_table, bt_row_stride: int, page_size: int,
                  t: int, positions, row: int = 0):
    """The scores of query token t at the given key positions only (the same
    formula as mqa_logits, for spot checks of long rows), and their error-bound
    magnitudes (as error_bound). Returns (scores float64, bound float64)."""
    pos = np.asarray(positions, dtype=np.int64)
    slots = P.slots_of(pos, np.full(pos.shape, row), block_table, bt_row_stride, page_size)
    qd = P.e4m3_decode(q_codes[t])                      # [H, D]
    kd = P.e4m3_decode(k_cache_fp8[slots])              # [n, D]
    ks = k_cache_scale[slots].astype(np.float64)
    w64 = np.asarray(w[t], np.float64)
    scores = ks * (w64 @ np.maximum(qd @ kd.T, 0.0))
    bound = ks * (np.abs(w64) @ (np.abs(qd) @ np.abs(kd).T))
    return scores, bound
