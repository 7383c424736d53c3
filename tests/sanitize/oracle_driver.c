/*
 * oracle_driver.c -- runs the CPU oracle (oracle/oracle_topk.c) under the
 * host address and undefined-behaviour sanitizers.
 *
 * Built and run by tests/test_sanitizers.py:
 *   gcc -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all \
 *       oracle/oracle_topk.c tests/sanitize/oracle_driver.c
 * Every row is cut to its exact valid length in its own heap block (the score
 * stride equals the row length, one row per call), so a read past the valid
 * prefix is a heap overflow that the sanitizer reports. Results are checked
 * against a brute-force rank count: position i is selected iff fewer than k
 * positions j < n have s_j > s_i, or s_j == s_i and j < i.
 * Prints "oracle sanitizer checks passed" and exits 0, or exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_topk_paged_rows(const float* scores, int64_t score_stride, const int32_t* lengths, int32_t row_begin,
                           int32_t row_end, const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                           int32_t k, int32_t* out_idx, int32_t* out_slots, int64_t out_stride);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {   /* xorshift64*, a test-input generator only */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int failures = 0;
#define CHECK(c, ...)                          \
  do {                                         \
    if (!(c)) {                                \
      fprintf(stderr, "FAIL: " __VA_ARGS__);   \
      fprintf(stderr, "\n");                   \
      ++failures;                              \
    }                                          \
  } while (0)

static int selected_by_rank(const float* s, int n, int k, int i) {
  int better = 0;
  for (int j = 0; j < n; ++j)
    if (s[j] > s[i] || (s[j] == s[i] && j < i)) ++better;
  return better < k;
}

static void one_case(int n, int k, int ps, int alphabet) {
  static const float vals[] = {0.0f, -0.0f, 1.5f, -2.0f, -INFINITY, 3.25f, 1e-30f, -1e30f};
  float* row = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) row[i] = vals[next_u32() % (uint32_t)alphabet];
  const int pages = n > 0 ? (n + ps - 1) / ps : 1;
  int32_t* table = (int32_t*)malloc(sizeof(int32_t) * (size_t)pages);
  for (int p = 0; p < pages; ++p) table[p] = pages - 1 - p;   /* reversed pages */
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  int32_t* slots = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  const int32_t len = n;
  const int rc = oracle_topk_paged_rows(row, n, &len, 0, 1, table, 0, ps, k, idx, slots, k);
  CHECK(rc == 0, "rc %d for n %d k %d", rc, n, k);
  const int m = n < k ? n : k;
  char* seen = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
  for (int j = 0; j < k; ++j) {
    if (j >= m) {
      CHECK(idx[j] == -1 && slots[j] == -1, "padding at %d (n %d k %d)", j, n, k);
      continue;
    }
    const int i = idx[j];
    CHECK(i >= 0 && i < n, "position %d out of [0, %d)", i, n);
    if (i < 0 || i >= n) continue;
    CHECK(!seen[i], "position %d twice", i);
    seen[i] = 1;
    CHECK(selected_by_rank(row, n, k, i), "position %d not in the top %d (n %d)", i, k, n);
    CHECK(slots[j] == table[i / ps] * ps + i % ps, "slot of position %d", i);
  }
  free(seen);
  free(slots);
  free(idx);
  free(table);
  free(row);
}

int main(void) {
  for (int t = 0; t < 400; ++t) {
    const int n = (int)(next_u32() % 300);
    const int k = 1 + (int)(next_u32() % 320);
    const int ps = 1 + (int)(next_u32() % 70);
    one_case(n, k, ps, 2 + (int)(next_u32() % 7));
  }
  one_case(0, 1, 64, 3);
  one_case(2048, 2048, 64, 8);
  one_case(2049, 2048, 64, 8);
  one_case(5000, 2048, 64, 2);

  /* rejected arguments and NaN inside the valid prefix */
  float r[3] = {1.0f, NAN, 2.0f};
  int32_t tab[1] = {0}, out_i[4], out_s[4];
  int32_t len3 = 3, len1 = 1, bad_len = -1;
  CHECK(oracle_topk_paged_rows(r, 3, &len3, 0, 1, tab, 0, 64, 2, out_i, out_s, 4) == -2, "NaN accepted");
  CHECK(oracle_topk_paged_rows(r, 3, &len1, 0, 1, tab, 0, 64, 1, out_i, out_s, 4) == 0, "NaN past len");
  CHECK(oracle_topk_paged_rows(NULL, 3, &len3, 0, 1, tab, 0, 64, 2, out_i, out_s, 4) == -1, "NULL scores");
  CHECK(oracle_topk_paged_rows(r, 3, &len3, 0, 1, tab, 0, 0, 2, out_i, out_s, 4) == -1, "page size 0");
  CHECK(oracle_topk_paged_rows(r, 3, &len3, 0, 1, tab, 0, 64, 0, out_i, out_s, 4) == -1, "k 0");
  CHECK(oracle_topk_paged_rows(r, 3, &len3, 0, 1, tab, 0, 64, 5, out_i, out_s, 4) == -1, "out stride < k");
  CHECK(oracle_topk_paged_rows(r, 3, &bad_len, 0, 1, tab, 0, 64, 1, out_i, out_s, 4) == -1, "negative length");
  CHECK(oracle_topk_paged_rows(r, 3, &len3, 1, 0, tab, 0, 64, 1, out_i, out_s, 4) == -1, "row range");

  if (failures) {
    fprintf(stderr, "%d oracle sanitizer checks failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer checks passed\n");
  return 0;
}
