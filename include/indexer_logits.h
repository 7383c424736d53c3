/*
 * indexer_logits.h -- C ABI of the indexer's score producer for MI355X
 * (gfx950): MQA logits of a few query tokens against the paged FP8 key
 * cache, in libsparse_topk.so next to the top-k selection that reads them.
 *
 * What it computes
 * ----------------
 * Passages: the lmsys.org page "Serving GLM5.2 NVFP4 Agentic Workload with
 * SGLang": section "Kernel Optimization / TopK-V2" (the DSA indexer turns each
 * query into FP32 scores over historical KV positions), section "Indexer
 * Prologue Fusion" (FP8 queries with head-gate scaling, FP8 keys in the paged
 * indexer cache) and section "What's Next" (the MQA logits kernel). The page
 * prints no formula; the library implements the lightning indexer's
 * published score on the quantized operands, with the positive scales
 * outside the ReLU:
 *
 *   out[t][s] = k_scale[slot(s)] * sum_h w[t][h] * ReLU( sum_d decode(q_codes[t][h][d])
 *                                                         * decode(k_fp8[slot(s)][d]) )
 *
 * for every query token t < tokens and key position s < min(lengths[t],
 * max_len); slot(s) = block_table[s / page_size] * page_size + s % page_size;
 * decode = FP8 E4M3 (OCP "fn"). w is the head-gate weight with the query
 * scale folded in (indexer_query_prologue's w_out); k_fp8 / k_scale are the
 * cache indexer_key_prologue fills. Dot products run on the matrix cores in
 * FP8 with FP32 accumulation, the head sum in FP32.
 *
 * Scope: the decode / verify regime, where one request's few query tokens
 * share every key: tokens * heads <= INDEXER_LOGITS_MAX_QROWS query rows,
 * heads 32, 64 or 128, D = 128, one request per call (block_table is that
 * request's row). Entries out[t][s] for s >= min(lengths[t], max_len) are
 * not written. Codes are finite E4M3 values: a score whose query or key
 * holds the NaN code (0x7F or 0xFF) is unspecified.
 *
 * Memory, threading, errors
 * -------------------------
 * DEVICE pointers; `stream` is a hipStream_t as void*; one kernel enqueued,
 * no allocation or synchronisation (graph-capturable). q_codes, w and k_fp8
 * must be 16-byte aligned. Host-checkable errors return TOPK_ERR_INVALID_ARG
 * (sizes, NULLs, alignment, out_stride < max_len) or TOPK_ERR_UNSUPPORTED
 * (too many query rows) and enqueue nothing. A table entry giving a slot
 * outside [0, num_slots) skips that key and sets INDEXER_DEVICE_BAD_SLOT in
 * *status (status may be NULL).
 */
#ifndef INDEXER_LOGITS_H
#define INDEXER_LOGITS_H

#include <stddef.h>
#include <stdint.h>

#include "indexer_prologue.h"
#include "sparse_topk.h"

#ifdef __cplusplus
extern "C" {
#endif

#define INDEXER_LOGITS_MAX_QROWS 512

/* MQA logits (see above). q_codes uint8 [tokens][heads][128]; w float
 * [tokens][heads]; k_fp8 uint8 [num_slots][128]; k_scale float [num_slots];
 * lengths int32 [tokens]; out float [tokens][out_stride]. Passage: lmsys page,
 * sections "Kernel Optimization / TopK-V2" and "What's Next". */
topk_status indexer_mqa_logits(const uint8_t* q_codes, const float* w, int32_t tokens, int32_t heads,
                               const uint8_t* k_fp8, const float* k_scale, int64_t num_slots,
                               const int32_t* block_table, int32_t page_size, const int32_t* lengths,
                               int32_t max_len, float* out, int64_t out_stride, int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INDEXER_LOGITS_H */
