/*
 * oracle_topk.c -- CPU oracle for indexer top-k selection with paged slot mapping.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file; only the tests, the package smoke check and the benchmark's CPU
 * baseline use it. It shares no code with the HIP library.
 *
 * What it computes (the plain definition, not the GPU method):
 *   The lmsys.org page "Serving GLM5.2 NVFP4 Agentic Workload with SGLang",
 *   section TopK-V2 (text and the captions of Figures 2 and 3), describes a
 *   kernel that, for each query row of FP32 indexer scores over historical KV
 *   positions, returns exactly k entries (runtime k up to 2048), resolves the
 *   boundary by exact FP32 comparison with an exact tie-break, and translates
 *   each selected logical position into a physical indexer-KV-cache slot.
 *   Because the FP16 histogram there only locates the boundary and the final
 *   decision is exact, the result equals the plain definition:
 *
 *     T_r = first min(k, len_r) of [0, len_r) ordered by
 *           (score descending, position ascending),
 *
 *   with ties at equal score going to the lower logical position (the tie rule
 *   is not printed on the page; "lower index first" is the reading adopted).
 *   Each selected position i maps to slot  bt[r][i / ps] * ps + i % ps.
 *
 * Steps, in order: (1) reject NaN inside the valid prefix; (2) build the
 * (score, position) pairs of the valid prefix only; (3) sort them with the
 * comparator above (IEEE comparison: -0.0 == +0.0, -inf is the lowest value);
 * (4) keep the first m = min(k, len); (5) map positions to slots in 64-bit
 * arithmetic and check the result fits int32; (6) write the m entries in
 * sorted order, then -1 up to k.
 *
 * Parity pins (outside this file, in tests/): brute-force rank counting,
 * exhaustive subsets on tiny rows, numpy's stable argsort, argmax for k = 1,
 * closed forms of the adversarial tie rows, and hand-built tie cases.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARG = -1,
  ORACLE_ERR_NAN = -2,
  ORACLE_ERR_SLOT = -3,
  ORACLE_ERR_NOMEM = -4,
};

typedef struct {
  float score;
  int32_t pos;
} scored_pos;

/* (score descending, position ascending): a total order on distinct positions. */
static int by_score_then_pos(const void* pa, const void* pb) {
  const scored_pos* a = (const scored_pos*)pa;
  const scored_pos* b = (const scored_pos*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->pos > b->pos) - (a->pos < b->pos);
}

/*
 * Rows [row_begin, row_end) of the batch.
 *   scores        float [rows][score_stride], row-major, host memory
 *   lengths       int32 [rows]
 *   block_table   int32; row r uses block_table + r * bt_stride (bt_stride 0: shared)
 *   out_idx       int32 [rows][out_stride] or NULL
 *   out_slots     int32 [rows][out_stride] or NULL
 * Returns 0, or a negative code; on error the row being processed is left
 * partially written.
 */
int oracle_topk_paged_rows(const float* scores, int64_t score_stride,
                           const int32_t* lengths, int32_t row_begin, int32_t row_end,
                           const int32_t* block_table, int64_t bt_stride,
                           int32_t page_size, int32_t k,
                           int32_t* out_idx, int32_t* out_slots, int64_t out_stride) {
  if (!scores || !lengths || !block_table || page_size < 1 || k < 1 ||
      out_stride < k || row_begin < 0 || row_end < row_begin || bt_stride < 0)
    return ORACLE_ERR_ARG;
  int64_t max_len = 0;
  for (int32_t r = row_begin; r < row_end; ++r) {
    if (lengths[r] < 0 || lengths[r] > score_stride) return ORACLE_ERR_ARG;
    if (lengths[r] > max_len) max_len = lengths[r];
  }
  scored_pos* pairs = (scored_pos*)malloc((size_t)(max_len > 0 ? max_len : 1) * sizeof(scored_pos));
  if (!pairs) return ORACLE_ERR_NOMEM;

  int rc = ORACLE_OK;
  for (int32_t r = row_begin; r < row_end && rc == ORACLE_OK; ++r) {
    const float* row = scores + (int64_t)r * score_stride;
    const int32_t* table = block_table + (int64_t)r * bt_stride;
    const int32_t n = lengths[r];
    for (int32_t i = 0; i < n; ++i) {
      if (isnan(row[i])) { rc = ORACLE_ERR_NAN; break; }
      pairs[i].score = row[i];
      pairs[i].pos = i;
    }
    if (rc != ORACLE_OK) break;
    qsort(pairs, (size_t)n, sizeof(scored_pos), by_score_then_pos);
    const int32_t m = n < k ? n : k;
    for (int32_t j = 0; j < k; ++j) {
      int32_t idx = -1, slot = -1;
      if (j < m) {
        idx = pairs[j].pos;
        const int64_t page = table[idx / page_size];
        const int64_t s = page * (int64_t)page_size + (int64_t)(idx % page_size);
        if (page < 0 || s > INT32_MAX) { rc = ORACLE_ERR_SLOT; break; }
        slot = (int32_t)s;
      }
      if (out_idx) out_idx[(int64_t)r * out_stride + j] = idx;
      if (out_slots) out_slots[(int64_t)r * out_stride + j] = slot;
    }
  }
  free(pairs);
  return rc;
}
