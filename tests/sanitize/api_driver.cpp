// api_driver.cpp -- calls every entry point of include/sparse_topk.h with
// host-checkable bad arguments, and valid configurations as far as the host
// code goes, in a build whose C ABI host code carries the address and
// undefined-behaviour sanitizers (sparse_attention_indexer_amd/build.py,
// build_api_sanitizer_driver). Without a GPU every valid configuration stops
// at the device query with TOPK_ERR_HIP; with one it may succeed. Nothing here
// launches a kernel on valid data: every call either fails its argument check
// or has no device to run on.
// Prints "api sanitizer checks passed" and exits 0, or exits 1.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "sparse_topk.h"

static int failures = 0;
#define CHECK(c, what)                            \
  do {                                            \
    if (!(c)) {                                   \
      std::fprintf(stderr, "FAIL: %s\n", what);   \
      ++failures;                                 \
    }                                             \
  } while (0)

static topk_config good() {
  topk_config c;
  std::memset(&c, 0, sizeof(c));
  c.k = 2048;
  c.max_rows = 7;
  c.max_len = 80000;
  return c;
}

int main() {
  size_t pb = 0, wb = 0;
  for (int s : {0, -1, -2, -3, -4, -5, -99}) CHECK(topk_status_string((topk_status)s) != nullptr, "status string");
  CHECK(std::strcmp(topk_status_string((topk_status)-99), "unknown status") == 0, "unknown status string");
  CHECK(topk_register_capacity() == 32768, "register capacity");
  CHECK(topk_stream_read_groups() >= 1, "stream read groups");

  // configurations rejected before any device query
  CHECK(topk_query_sizes(nullptr, &pb, &wb) == TOPK_ERR_INVALID_ARG, "NULL cfg");
  topk_config c = good();
  CHECK(topk_query_sizes(&c, nullptr, &wb) == TOPK_ERR_INVALID_ARG, "NULL plan size");
  const struct {
    const char* what;
    void (*edit)(topk_config&);
  } bad[] = {
      {"k 0", [](topk_config& x) { x.k = 0; }},
      {"k 2049", [](topk_config& x) { x.k = 2049; }},
      {"max_rows 0", [](topk_config& x) { x.max_rows = 0; }},
      {"max_len -1", [](topk_config& x) { x.max_len = -1; }},
      {"max_len 2^31", [](topk_config& x) { x.max_len = int64_t(1) << 31; }},
      {"force_path 4", [](topk_config& x) { x.force_path = 4; }},
      {"wg_per_row 1", [](topk_config& x) { x.wg_per_row = 1; }},
      {"cand_capacity -1", [](topk_config& x) { x.cand_capacity = -1; }},
      {"min_chunk -1", [](topk_config& x) { x.min_chunk = -1; }},
      {"spin_limit -2", [](topk_config& x) { x.spin_limit = -2; }},
      {"reserved", [](topk_config& x) { x.reserved[1] = 3; }},
  };
  for (const auto& b : bad) {
    topk_config x = good();
    b.edit(x);
    CHECK(topk_query_sizes(&x, &pb, &wb) == TOPK_ERR_INVALID_ARG, b.what);
    CHECK(topk_plan(&x, nullptr, 1, nullptr, 0, nullptr) == TOPK_ERR_INVALID_ARG, b.what);
    CHECK(topk_select_paged(&x, nullptr, nullptr, 0, nullptr, 1, nullptr, 0, 64, nullptr, nullptr, 2048, nullptr, 0,
                            nullptr) == TOPK_ERR_INVALID_ARG,
          b.what);
    CHECK(topk_select_paged_noalloc(&x, nullptr, 0, nullptr, 1, nullptr, 0, 64, nullptr, nullptr, 2048, nullptr,
                                    nullptr) == TOPK_ERR_INVALID_ARG,
          b.what);
  }
  {
    topk_config x = good();
    const topk_status n = topk_select_paged_noalloc(&x, nullptr, 80000, nullptr, 7, nullptr, 0, 64, nullptr, nullptr,
                                                    2048, nullptr, nullptr);
    CHECK(n == TOPK_ERR_HIP || n == TOPK_ERR_INVALID_ARG, "no-alloc call with NULL buffers");
  }
  topk_config reg = good();
  reg.force_path = TOPK_PATH_REGISTER;
  reg.max_len = 32769;
  CHECK(topk_query_sizes(&reg, &pb, &wb) == TOPK_ERR_UNSUPPORTED, "register path too long");

  // valid configurations reach the device query
  c = good();
  const topk_status q = topk_query_sizes(&c, &pb, &wb);
  CHECK(q == TOPK_ERR_HIP || q == TOPK_OK, "valid configuration");
  const topk_status p = topk_plan(&c, nullptr, 7, nullptr, 0, nullptr);
  CHECK(p == TOPK_ERR_HIP || p == TOPK_ERR_INVALID_ARG, "plan without buffers");
  const topk_status t = topk_select_paged_timed(&c, nullptr, nullptr, 0, nullptr, 7, nullptr, 0, 64, nullptr,
                                                nullptr, 2048, nullptr, 0, nullptr, nullptr, nullptr);
  CHECK(t == TOPK_ERR_INVALID_ARG, "timed call without events");

  // the other entry points' argument checks
  CHECK(topk_workspace_init(nullptr, 256, nullptr) == TOPK_ERR_INVALID_ARG, "workspace NULL");
  int32_t word = 0;
  CHECK(topk_workspace_init(&word, 3, nullptr) == TOPK_ERR_INVALID_ARG, "workspace bytes % 4");
  CHECK(topk_read_status(nullptr, 256, &word, nullptr) == TOPK_ERR_INVALID_ARG, "status NULL");
  CHECK(topk_read_status(&word, 16, &word, nullptr) == TOPK_ERR_INVALID_ARG, "status too small");
  CHECK(topk_debug_keys(nullptr, 5, nullptr, nullptr, nullptr) == TOPK_ERR_INVALID_ARG, "debug keys NULL");
  CHECK(topk_debug_keys(nullptr, -1, nullptr, nullptr, nullptr) == TOPK_ERR_INVALID_ARG, "debug keys n < 0");
  float f[8] = {0};
  CHECK(topk_debug_stream_read(nullptr, 8, nullptr, nullptr, nullptr, nullptr) == TOPK_ERR_INVALID_ARG,
        "stream read NULL");
  CHECK(topk_debug_stream_read(f + 1, 4, f, nullptr, nullptr, nullptr) == TOPK_ERR_INVALID_ARG ||
            (reinterpret_cast<uintptr_t>(f + 1) % 16) == 0,
        "stream read misaligned");
  CHECK(topk_debug_stream_read(f, 8, f, nullptr, &word, nullptr) == TOPK_ERR_INVALID_ARG, "one event");
  CHECK(topk_debug_histogram(nullptr, 0, nullptr, 3, 2048, nullptr, nullptr, nullptr) == TOPK_ERR_INVALID_ARG,
        "histogram NULL");
  CHECK(topk_debug_histogram(f, 8, nullptr, 0, 0, nullptr, nullptr, nullptr) == TOPK_ERR_INVALID_ARG,
        "histogram k 0");
  CHECK(topk_debug_histogram(f, -1, nullptr, 0, 5, nullptr, nullptr, nullptr) == TOPK_ERR_INVALID_ARG,
        "histogram stride");

  if (failures) {
    std::fprintf(stderr, "%d api sanitizer checks failed\n", failures);
    return 1;
  }
  std::printf("api sanitizer checks passed\n");
  return 0;
}
