/*
 * indexer_prologue.h -- C ABI of the fused indexer key prologue for MI355X
 * (gfx950), in the same library as the top-k selection (libsparse_topk.so).
 *
 * What it computes
 * ----------------
 * Passage: the lmsys.org page "Serving GLM5.2 NVFP4 Agentic Workload with
 * SGLang", section "Indexer Prologue Fusion" (text and Figure 5). The key
 * half of the fused BF16 projection feeds one kernel that applies LayerNorm,
 * RoPE and FP8 quantization and stores the result into the paged indexer KV
 * cache, with no Hadamard transform. The page names these steps but prints
 * no formula; the library implements these readings:
 *
 *   x      = the token's D = 128 BF16 key activations, as FP32;
 *   y      = (x - mean(x)) / sqrt(var(x) + eps) * ln_weight + ln_bias
 *            (biased variance);
 *   rotary on dims [0, rope_dim), interleaved pairs (2i, 2i+1):
 *            (a, b) -> (a c - b s, a s + b c),  c = cos_sin[pos][i],
 *            s = cos_sin[pos][rope_dim / 2 + i]  (the caller's rotary cache);
 *   amax   = max |y| over the token, floored at 2^-64;
 *   codes  = FP8 E4M3 (OCP "fn": bias 7, largest finite 448) of
 *            y * (448 / amax), rounded to nearest even, saturated at +-448;
 *   scale  = amax / 448  (so y ~ decode(code) * scale);
 *   slot   = block_table[row * bt_row_stride + pos / page_size] * page_size
 *            + pos % page_size  (the top-k library's slot formula);
 *   cache_fp8[slot * 128 + d] = codes[d],  cache_scale[slot] = scale.
 *
 * Every step runs in FP32 on the device (the quantization's FP32 division and
 * products exactly as written above).
 *
 * Memory and threading
 * --------------------
 * All data pointers are DEVICE pointers; `stream` is a hipStream_t passed as
 * void* (NULL: the default stream). The call enqueues one kernel and never
 * allocates, frees or synchronises, so it may be captured into a HIP graph.
 * The caller owns every buffer.
 *
 * Layouts
 *   k_act        uint16 (BF16 bits) [num_tokens][k_stride], k_stride >= 128 and
 *                a multiple of 8, base 16-byte aligned;
 *   ln_weight, ln_bias  float [128];
 *   cos_sin      float [max_pos][rope_dim], 16-byte aligned (unused when
 *                rope_dim == 0);
 *   positions    int32 [num_tokens];  token_row int32 [num_tokens] or NULL
 *                (every token in row 0); a negative row marks a padding token,
 *                which stores nothing;
 *   block_table  int32, row r at block_table + r * bt_row_stride (0: one
 *                table shared by all rows);
 *   cache_fp8    uint8 [num_slots][128], 16-byte aligned; cache_scale float
 *                [num_slots];
 *   status       int32, one word the kernel ORs INDEXER_DEVICE_* flags into,
 *                or NULL.
 *
 * Errors
 * ------
 * Host-checkable arguments are checked synchronously (TOPK_ERR_INVALID_ARG,
 * nothing enqueued): NULL required pointers, dim != 128, rope_dim not a
 * multiple of 8 in [0, 128], page_size < 1, max_pos < 1, num_tokens < 0,
 * k_stride, alignments, num_slots < 1, eps not finite or negative, reserved
 * fields not zero. A launch failure returns TOPK_ERR_HIP. Device data is
 * checked per token: a position outside [0, max_pos) or a slot outside
 * [0, num_slots) skips the token's store and sets a flag in *status.
 */
#ifndef INDEXER_PROLOGUE_H
#define INDEXER_PROLOGUE_H

#include <stddef.h>
#include <stdint.h>

#include "sparse_topk.h"

#ifdef __cplusplus
extern "C" {
#endif

#define INDEXER_KEY_DIM 128

/* Flags the key prologue ORs into its status word. */
#define INDEXER_DEVICE_BAD_POSITION 0x100  /* a position outside [0, max_pos) */
#define INDEXER_DEVICE_BAD_SLOT 0x200      /* a slot outside [0, num_slots) */

typedef struct {
  int32_t dim;          /* head dimension: 128 */
  int32_t rope_dim;     /* rotated leading dims: a multiple of 8 in [0, dim] */
  float eps;            /* LayerNorm epsilon, finite, >= 0 */
  int32_t page_size;    /* tokens per cache page, >= 1 */
  int32_t max_pos;      /* rows of cos_sin (positions must be below it), >= 1 */
  int32_t reserved[3];  /* must be zero */
} indexer_key_config;

/* The fused key path for num_tokens tokens (see above). Passage: lmsys page,
 * section "Indexer Prologue Fusion", key path. */
topk_status indexer_key_prologue(const indexer_key_config* cfg, const uint16_t* k_act, int64_t k_stride,
                                 int32_t num_tokens, const float* ln_weight, const float* ln_bias,
                                 const float* cos_sin, const int32_t* positions, const int32_t* token_row,
                                 const int32_t* block_table, int64_t bt_row_stride, uint8_t* cache_fp8,
                                 float* cache_scale, int64_t num_slots, int32_t* status, void* stream);

/* The fused query path for tokens x heads rows of 128 dims (lmsys page,
 * section "Indexer Prologue Fusion", query path: RoPE + FP8 quantization +
 * head-gate scaling). Per (token t, head h):
 *   y      = rotary of the BF16 row q_act[t][h] at positions[t] (as the key path;
 *            rope_dim 0 skips it);
 *   amax   = max |y| floored at 2^-64; codes = E4M3 RNE of y * (448 / amax);
 *   w_out[t][h] = (w_raw[t][h] * (amax / 448)) * gate_scale  (FP32, in that order):
 *            the query scale is folded into the head-gate weight, which is
 *            exact under the indexer's ReLU since the scale is positive.
 * Layouts: q_act uint16 [tokens][heads][128] and q_codes uint8 [tokens][heads][128]
 * (16-byte aligned), w_raw / w_out float [tokens][heads], positions int32
 * [tokens], cos_sin as for the key path (max_pos rows). Errors: bad sizes,
 * NULLs, alignment, gate_scale <= 0 or not finite -> TOPK_ERR_INVALID_ARG;
 * a position outside [0, max_pos) (with rope_dim > 0) skips the row and sets
 * INDEXER_DEVICE_BAD_POSITION in *status (status may be NULL). */
topk_status indexer_query_prologue(const uint16_t* q_act, int32_t tokens, int32_t heads, const float* w_raw,
                                   float gate_scale, const float* cos_sin, int32_t rope_dim, int32_t max_pos,
                                   const int32_t* positions, uint8_t* q_codes, float* w_out, int32_t* status,
                                   void* stream);

/* Test hook: the kernel's own FP32 -> E4M3 conversion (saturating, round to
 * nearest even) of n values, x[i] -> out[i]. Passage: none (a window on the
 * quantizer of indexer_key_prologue). */
topk_status indexer_debug_fp8(const float* x, int64_t n, uint8_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INDEXER_PROLOGUE_H */
