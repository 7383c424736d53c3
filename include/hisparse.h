/*
 * hisparse.h -- C ABI of the HiSparse top-k resolver for MI355X (gfx950), in
 * libsparse_topk.so next to the top-k selection whose output it consumes.
 *
 * What it computes
 * ----------------
 * Passage: the vllm.ai page "GLM 5.3 Optimizations, Part 1: Hybrid HiSparse
 * Offloading in vLLM", section "How it works" (mixed residency) and the
 * hot-buffer size it states (2x top-K rows per request). One kernel maps
 * every selected token of a decode step to the KV-tensor row the sparse
 * attention reads: a token on a resident page is read in place, a token in
 * the request's hot buffer is read there and its LRU entry refreshed, and a
 * miss copies its row from pinned host memory into a least-recently-used hot
 * slot. No host decision is on the path, so the call can be captured into a
 * HIP graph. The page gives no victim rule or layout; the library implements:
 *
 *   for request r, selected position p (sel[r][j], -1 = none):
 *     page = block_table[r][p / page_size];
 *     page >= 0            -> row = page * page_size + p % page_size;
 *     map[r][p] = s >= 0   -> row = hot_rows[r][s], stamp[r][s] = step;
 *     otherwise a miss.
 *   Misses are served in increasing position order. The victims are the slots
 *   whose stamp is not `step`, least recently used first (smaller stamp),
 *   ties by lower slot index. Miss i takes victim i: map[r][tag[r][v]] = -1
 *   (if tagged), tag[r][v] = p, map[r][p] = v, stamp[r][v] = step, the host row
 *   host_table[r][p / page_size] * page_size + p % page_size of host_pool is
 *   copied to KV row hot_rows[r][v], and row = hot_rows[r][v]. With fewer
 *   victims than misses the remaining (highest) positions get row -1 and
 *   HISPARSE_DEVICE_HOT_FULL is set.
 *   rows_out[r][j] = row (int64), -1 for sel -1.
 *
 * `step` must exceed every stamp stored so far (stamps start at 0 = never
 * used); the selected positions of a request must be distinct (a top-k row).
 *
 * Memory and threading
 * --------------------
 * Device pointers except host_pool, which is pinned host memory (allocated
 * with hipHostMalloc, or a pinned torch tensor); the library checks with
 * hipPointerGetAttributes that it is host memory mapped for the device and
 * reads it through the device mapping. One workgroup per request; requests'
 * hot rows must be disjoint KV rows. `stream` is a hipStream_t as void*; one
 * kernel, no allocation or synchronisation. Calls that share state arrays
 * must not run concurrently.
 *
 * Layouts: sel int32 [requests][sel_stride] (k used); block_table and
 * host_table int32 [requests][*_stride] covering ceil(max_ctx / page_size)
 * pages; hot_rows int64 [requests][hot]; tag int32 and stamp uint32
 * [requests][hot]; map int32 [requests][max_ctx]; kv uint8 [kv_rows][row_bytes];
 * host_pool uint8 [host_rows][row_bytes] (host_rows < 2^31); rows_out int64 [requests][k].
 *
 * Errors: host-checkable arguments -> TOPK_ERR_INVALID_ARG (k outside
 * [1, 2048], hot outside [1, 4096], page_size < 1, max_ctx < 1, row_bytes not a
 * positive multiple of 16, strides below k or the page count, NULL pointers,
 * misaligned kv or host_pool, host_pool not pinned host memory, step 0).
 * Device data: a position outside [0, max_ctx), a hot row outside the KV
 * tensor or a host row outside the pool skips that token (row -1) and sets
 * HISPARSE_DEVICE_BAD_INDEX in *status (status may be NULL).
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#include "sparse_topk.h"

#ifdef __cplusplus
extern "C" {
#endif

#define HISPARSE_DEVICE_HOT_FULL 0x1000   /* more misses than evictable hot slots */
#define HISPARSE_DEVICE_BAD_INDEX 0x2000  /* a position, hot row or host row out of range */

typedef struct {
  int32_t k;          /* selected positions per request, 1..2048 */
  int32_t hot;        /* hot slots per request, 1..4096 */
  int32_t page_size;  /* tokens per page, >= 1 */
  int32_t max_ctx;    /* positions per request (entries of map), >= 1 */
  int32_t row_bytes;  /* bytes per KV row, a positive multiple of 16 */
  int32_t reserved[3];/* must be zero */
} hisparse_config;

/* One decode step of the resolver for `requests` requests (see above).
 * Passage: vllm.ai page, section "How it works", mixed residency. */
topk_status hisparse_resolve(const hisparse_config* cfg, uint32_t step, int32_t requests, const int32_t* sel,
                             int64_t sel_stride, const int32_t* block_table, int64_t bt_stride,
                             const int32_t* host_table, int64_t host_bt_stride, const int64_t* hot_rows,
                             int32_t* tag, uint32_t* stamp, int32_t* map, uint8_t* kv, int64_t kv_rows,
                             const uint8_t* host_pool, int64_t host_rows, int64_t* rows_out, int32_t* status,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
