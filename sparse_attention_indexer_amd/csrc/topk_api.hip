// topk_api.hip -- C ABI of the indexer top-k library: argument checks, buffer
// sizing and kernel launches. No allocation and no synchronisation happen
// here except in topk_read_status, which says so.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "sparse_topk.h"
#include "topk_layout.hpp"
#include "topk_plan.hpp"

static_assert(satopk::kInKernelPlanRows == TOPK_IN_KERNEL_PLAN_ROWS, "header and kernels agree");
static_assert(satopk::kInKernelPlanRows <= satopk::kBlock, "one row per thread");

namespace satopk {
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int grid, bool vec, bool stream_items, int overlap, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop);
hipError_t launch_fill(void* p, size_t bytes, hipStream_t s);
hipError_t launch_debug_keys(const float* x, int64_t n, uint32_t* bin, uint32_t* k32, hipStream_t s);
hipError_t select_occupancy(int* per_cu);
hipError_t launch_stream_read(const float* x, int64_t n, float* out, hipStream_t s, hipEvent_t start,
                              hipEvent_t stop);
int stream_read_groups();
hipError_t launch_debug_hist(const float* scores, int64_t stride, const int32_t* lengths, int32_t rows, int32_t k,
                             uint32_t* hist, uint32_t* res, hipStream_t s);
}  // namespace satopk

using namespace satopk;

namespace {

// Per-device CU count and co-resident selection workgroups per CU. This cache
// is the library's only global state; it never changes once filled. Filled
// under a lock once per device; every later call reads it without one (the
// release store of `ready` publishes the two counts).
struct DevInfo {
  int cus = 0;
  int per_cu = 0;
};
struct DevSlot {
  std::atomic<bool> ready{false};
  DevInfo info;
};
constexpr int kMaxDevices = 64;
DevSlot g_dev[kMaxDevices];
std::mutex g_dev_mu;

topk_status device_info(DevInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TOPK_ERR_HIP;
  DevSlot& d = g_dev[dev];
  if (!d.ready.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_dev_mu);
    if (!d.ready.load(std::memory_order_relaxed)) {
      int cus = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return TOPK_ERR_HIP;
      int per_cu = 0;
      if (select_occupancy(&per_cu) != hipSuccess || per_cu <= 0) return TOPK_ERR_HIP;
      d.info.cus = cus;
      d.info.per_cu = per_cu;
      d.ready.store(true, std::memory_order_release);
    }
  }
  *out = d.info;
  return TOPK_OK;
}

topk_status check_config(const topk_config* cfg) {
  if (!cfg) return TOPK_ERR_INVALID_ARG;
  if (cfg->k < 1 || cfg->k > kMaxK) return TOPK_ERR_INVALID_ARG;
  if (cfg->max_rows < 1) return TOPK_ERR_INVALID_ARG;
  if (cfg->max_len < 0 || cfg->max_len > 0x7FFFFFFFLL) return TOPK_ERR_INVALID_ARG;
  if (cfg->force_path < TOPK_PATH_AUTO || cfg->force_path > TOPK_PATH_MULTI) return TOPK_ERR_INVALID_ARG;
  if (cfg->wg_per_row < 0 || cfg->wg_per_row == 1) return TOPK_ERR_INVALID_ARG;
  if (cfg->cand_capacity < 0 || cfg->min_chunk < 0) return TOPK_ERR_INVALID_ARG;
  if (cfg->spin_limit < -1) return TOPK_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (cfg->reserved[i] != 0) return TOPK_ERR_INVALID_ARG;
  if (cfg->force_path == TOPK_PATH_REGISTER && cfg->max_len > kTile) return TOPK_ERR_UNSUPPORTED;
  return TOPK_OK;
}

topk_status sizing(const topk_config* cfg, Sizing* s) {
  topk_status st = check_config(cfg);
  if (st != TOPK_OK) return st;
  DevInfo d;
  st = device_info(&d);
  if (st != TOPK_OK) return st;
  // The persistent grid: every co-resident workgroup, but no more than the
  // configuration can use (rows x chunks of a longest row), so small batches
  // launch few workgroups.
  const int64_t min_chunk = cfg->min_chunk > 0 ? cfg->min_chunk : kDefaultMinChunk;
  int64_t per_row = (cfg->max_len + min_chunk - 1) / min_chunk;
  if (cfg->force_path == TOPK_PATH_MULTI && per_row < 2) per_row = 2;
  if (cfg->wg_per_row > per_row) per_row = cfg->wg_per_row;
  if (per_row < 1) per_row = 1;
  const int64_t want = (int64_t)cfg->max_rows * per_row;
  int64_t cap = (int64_t)d.cus * d.per_cu;
  if (cap > kMaxRowGroups) cap = kMaxRowGroups;   // (a split row's vote counts its workgroups in 9 bits)
  s->grid = (int)(want < cap ? want : cap);
  s->max_items = s->grid + cfg->max_rows;
  int groups = s->grid / 2;
  if (groups > cfg->max_rows) groups = cfg->max_rows;
  if (groups < 1) groups = 1;
  s->max_groups = groups;
  const int64_t cand = cfg->cand_capacity > 0 ? cfg->cand_capacity
                                             : (cfg->max_len < kDefaultCandCap ? cfg->max_len : kDefaultCandCap);
  // even, so that every row's candidate slab starts on a 16-byte boundary
  // (the slabs are copied to LDS 16 bytes per lane)
  s->cand_cap = cand < 2 ? 2 : (cand + 1) / 2 * 2;
  const bool splits = cfg->force_path == TOPK_PATH_AUTO || cfg->force_path == TOPK_PATH_MULTI;
  // every row split needs its own group state and at least two workgroups of one grid round
  if (cfg->force_path == TOPK_PATH_MULTI && (int64_t)cfg->max_rows * 2 > s->grid) return TOPK_ERR_UNSUPPORTED;
  if (splits && cfg->wg_per_row > 0) {
    // a fixed group size must fit one grid round for every row at once
    if ((int64_t)cfg->wg_per_row * cfg->max_rows > s->grid || cfg->max_rows > s->max_groups)
      return TOPK_ERR_UNSUPPORTED;
  }
  s->plan_bytes = sizeof(PlanHeader) + sizeof(WorkItem) * (size_t)s->max_items;
  s->workspace_bytes = ws_total_bytes(*s);
  return TOPK_OK;
}

// Whether some work item can exceed one register tile. With the planner's
// defaults every row longer than a tile gets at least one workgroup per tile
// when the rows' tile counts fit the grid, which max_rows * ceil(max_len /
// tile) bounds. Forced paths and fixed group sizes can still produce longer
// items, and so can a minimum chunk above half a tile: the cap of
// floor(len / min_chunk) workgroups can then fall below ceil(len / tile)
// (at len = 80,000 and min_chunk = 32,768: 2 workgroups, chunks of 40,192).
// At or below half a tile, floor(len / min_chunk) >= floor(2 len / tile)
// >= ceil(len / tile) for every len above a tile.
bool items_may_stream(const topk_config* cfg, const Sizing& s) {
  if (cfg->max_len <= kTile) return false;
  if (cfg->force_path == TOPK_PATH_REGISTER) return false;   // max_len <= kTile is enforced
  if (cfg->force_path != TOPK_PATH_AUTO || cfg->wg_per_row > 0 || cfg->min_chunk > kTile / 2) return true;
  const int64_t tiles = (cfg->max_len + kTile - 1) / kTile;
  return (int64_t)cfg->max_rows * tiles > s.grid;
}

}  // namespace

extern "C" {

topk_status topk_query_sizes(const topk_config* cfg, size_t* plan_bytes, size_t* workspace_bytes) {
  if (!plan_bytes || !workspace_bytes) return TOPK_ERR_INVALID_ARG;
  Sizing s;
  const topk_status st = sizing(cfg, &s);
  if (st != TOPK_OK) return st;
  *plan_bytes = s.plan_bytes;
  *workspace_bytes = s.workspace_bytes;
  return TOPK_OK;
}

topk_status topk_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes % 4 != 0) return TOPK_ERR_INVALID_ARG;
  return launch_fill(workspace, workspace_bytes, (hipStream_t)stream) == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

topk_status topk_plan(const topk_config* cfg, const int32_t* lengths, int32_t num_rows, void* plan,
                      size_t plan_bytes, void* stream) {
  Sizing s;
  const topk_status st = sizing(cfg, &s);
  if (st != TOPK_OK) return st;
  if (num_rows < 0 || num_rows > cfg->max_rows || !plan) return TOPK_ERR_INVALID_ARG;
  if (num_rows > 0 && !lengths) return TOPK_ERR_INVALID_ARG;
  if (plan_bytes < s.plan_bytes) return TOPK_ERR_BUFFER_TOO_SMALL;
  if (num_rows <= kInKernelPlanRows && s.grid < 4096) return TOPK_OK;   // the selection kernel plans these itself
  const bool no_split = cfg->force_path == TOPK_PATH_REGISTER || cfg->force_path == TOPK_PATH_SINGLE;
  PlanArgs a;
  a.lengths = lengths;
  a.num_rows = num_rows;
  a.k = cfg->k;
  a.grid = s.grid;
  a.max_groups = s.max_groups;
  a.max_items = s.max_items;
  a.force_path = cfg->force_path;
  a.wg_per_row = no_split ? 0 : cfg->wg_per_row;
  a.min_chunk = cfg->min_chunk;
  a.max_len = cfg->max_len;
  a.header = (PlanHeader*)plan;
  a.items = (WorkItem*)((char*)plan + sizeof(PlanHeader));
  return launch_plan(a, (hipStream_t)stream) == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

}  // extern "C"

namespace {

// Host-checkable arguments of a selection call (beyond the configuration).
bool select_args_ok(const topk_config* cfg, int64_t score_row_stride, int32_t num_rows, const float* scores,
                    const int32_t* lengths, const int32_t* block_table, int64_t bt_row_stride, int32_t page_size,
                    const int32_t* out_slots, int64_t out_row_stride) {
  if (num_rows < 0 || num_rows > cfg->max_rows) return false;
  if (page_size < 1 || bt_row_stride < 0 || out_row_stride < cfg->k) return false;
  if (score_row_stride < cfg->max_len || score_row_stride < 0) return false;
  if (num_rows > 0 && (!scores || !lengths || !block_table || !out_slots)) return false;
  return true;
}

topk_status select_impl(const topk_config* cfg, const void* plan, const float* scores, int64_t score_row_stride,
                        const int32_t* lengths, int32_t num_rows, const int32_t* block_table, int64_t bt_row_stride,
                        int32_t page_size, int32_t* out_slots, int32_t* out_indices, int64_t out_row_stride,
                        void* workspace, size_t workspace_bytes, void* stream, void* start_event,
                        void* stop_event, int32_t* device_status = nullptr) {
  Sizing s;
  const topk_status st = sizing(cfg, &s);
  if (st != TOPK_OK) return st;
  if (!select_args_ok(cfg, score_row_stride, num_rows, scores, lengths, block_table, bt_row_stride, page_size,
                      out_slots, out_row_stride))
    return TOPK_ERR_INVALID_ARG;
  if ((!plan && (num_rows > kInKernelPlanRows || s.grid >= 4096)) || !workspace) return TOPK_ERR_INVALID_ARG;
  if (workspace_bytes < s.workspace_bytes) return TOPK_ERR_BUFFER_TOO_SMALL;
  if (num_rows == 0) return TOPK_OK;
  SelectArgs a;
  a.scores = scores;
  a.stride = score_row_stride;
  a.lengths = lengths;
  a.num_rows = num_rows;
  a.k = cfg->k;
  a.table = block_table;
  a.table_stride = bt_row_stride;
  a.page_size = page_size;
  a.page_shift = -1;
  if ((page_size & (page_size - 1)) == 0) {
    int sh = 0;
    while ((1 << sh) < page_size) ++sh;
    a.page_shift = sh;
  }
  a.out_slots = out_slots;
  a.out_idx = out_indices;
  a.out_stride = out_row_stride;
  const bool here = num_rows <= kInKernelPlanRows && s.grid < 4096;   // the in-kernel scan packs 12-bit item counts
  a.plan = here ? nullptr : (const PlanHeader*)plan;
  a.items = here ? nullptr : (const WorkItem*)((const char*)plan + sizeof(PlanHeader));
  a.force_path = cfg->force_path;
  a.wg_per_row = (cfg->force_path == TOPK_PATH_REGISTER || cfg->force_path == TOPK_PATH_SINGLE) ? 0 : cfg->wg_per_row;
  a.min_chunk = cfg->min_chunk;
  a.max_groups = s.max_groups;
  a.groups = (GroupState*)((char*)workspace + ws_group_offset());
  a.cand = (uint64_t*)((char*)workspace + ws_cand_offset(s));
  a.cand_cap = s.cand_cap;
  a.status = device_status ? device_status : (int32_t*)workspace;
  a.max_len = cfg->max_len;
  a.spin_limit = cfg->spin_limit == 0 ? kDefaultSpinLimit : cfg->spin_limit < 0 ? 0u : (uint32_t)cfg->spin_limit;
  // The selection kernel starts loading its tile before the lengths arrive,
  // guessing that every row has max_len scores; the guess is the planner's
  // own split of such a batch.
  a.guess_groups = 1;
  a.guess_chunk = cfg->max_len;
  if (here) {
    PlanArgs p{};
    p.num_rows = num_rows;
    p.k = cfg->k;
    p.grid = s.grid;
    p.max_groups = s.max_groups;
    p.force_path = a.force_path;
    p.wg_per_row = a.wg_per_row;
    p.min_chunk = a.min_chunk;
    p.max_len = cfg->max_len;
    const int32_t L = (int32_t)cfg->max_len;
    const bool longer = L > split_floor(p);
    const uint64_t total = longer ? (uint64_t)L * (uint64_t)num_rows : 0ull;
    const uint32_t tiles = longer ? (uint32_t)(tiles_of(L) * num_rows) : 0u;
    int64_t c = L;
    a.guess_groups = split_of(L, p, total, longer ? num_rows : 0, tiles, &c);
    a.guess_chunk = c;
  }
  const bool vec = ((uintptr_t)scores % 16 == 0) && (score_row_stride % 4 == 0);
  // The planning overlaps the guessed tile's loads when that tile is at least
  // half a tile long (all 16 vector groups) or at most 8,192 scores (the
  // first 4).
  const int64_t guess_len = a.guess_groups > 1 ? a.guess_chunk : cfg->max_len;
  const int overlap = !here ? 0 : (guess_len >= kTile / 2 && guess_len <= kTile) ? 16 : (guess_len <= 4 * kBlock * 4) ? 4 : 0;
  return launch_select(a, s.grid, vec, items_may_stream(cfg, s), overlap, (hipStream_t)stream, (hipEvent_t)start_event,
                       (hipEvent_t)stop_event) ==
                 hipSuccess
             ? TOPK_OK
             : TOPK_ERR_HIP;
}

}  // namespace

extern "C" {

topk_status topk_select_paged(const topk_config* cfg, const void* plan, const float* scores,
                              int64_t score_row_stride, const int32_t* lengths, int32_t num_rows,
                              const int32_t* block_table, int64_t bt_row_stride, int32_t page_size,
                              int32_t* out_slots, int32_t* out_indices, int64_t out_row_stride, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return select_impl(cfg, plan, scores, score_row_stride, lengths, num_rows, block_table, bt_row_stride, page_size,
                     out_slots, out_indices, out_row_stride, workspace, workspace_bytes, stream, nullptr, nullptr);
}

topk_status topk_select_paged_timed(const topk_config* cfg, const void* plan, const float* scores,
                                    int64_t score_row_stride, const int32_t* lengths, int32_t num_rows,
                                    const int32_t* block_table, int64_t bt_row_stride, int32_t page_size,
                                    int32_t* out_slots, int32_t* out_indices, int64_t out_row_stride,
                                    void* workspace, size_t workspace_bytes, void* stream, void* start_event,
                                    void* stop_event) {
  if (!start_event || !stop_event) return TOPK_ERR_INVALID_ARG;
  return select_impl(cfg, plan, scores, score_row_stride, lengths, num_rows, block_table, bt_row_stride, page_size,
                     out_slots, out_indices, out_row_stride, workspace, workspace_bytes, stream, start_event,
                     stop_event);
}

topk_status topk_read_status(const void* workspace, size_t workspace_bytes, int32_t* host_status, void* stream) {
  if (!workspace || !host_status || workspace_bytes < kStatusBytes) return TOPK_ERR_INVALID_ARG;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
    return TOPK_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TOPK_ERR_HIP;
  *host_status = v;
  return v ? TOPK_ERR_DEVICE : TOPK_OK;
}

int64_t topk_register_capacity(void) { return kTile; }

}  // extern "C"

// ---------------------------------------------------------------------------
// The library-owned workspace of topk_select_paged_noalloc: one array per
// device (each GPU holds its own copy for the life of the process). Host code
// never uses the array's name as an address; it uses the per-device pointer
// from hipGetSymbolAddress.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;   // TOPK_NOALLOC_SCRATCH_BYTES
static_assert(kNoAllocScratchBytes == TOPK_NOALLOC_SCRATCH_BYTES, "header and library agree");

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The calling thread's current device's copy of `scratch`, looked up once per
// device (with that device current).
topk_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TOPK_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TOPK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TOPK_OK;
}

}  // namespace

extern "C" {

topk_status topk_select_paged_noalloc(const topk_config* cfg, const float* scores, int64_t score_row_stride,
                                      const int32_t* lengths, int32_t num_rows, const int32_t* block_table,
                                      int64_t bt_row_stride, int32_t page_size, int32_t* out_slots,
                                      int32_t* out_indices, int64_t out_row_stride, int32_t* device_status,
                                      void* stream) {
  Sizing s;
  topk_status st = sizing(cfg, &s);
  if (st != TOPK_OK) return st;
  if (!select_args_ok(cfg, score_row_stride, num_rows, scores, lengths, block_table, bt_row_stride, page_size,
                      out_slots, out_row_stride))
    return TOPK_ERR_INVALID_ARG;
  if (num_rows > kInKernelPlanRows || s.grid >= 4096) return TOPK_ERR_UNSUPPORTED;   // needs a plan buffer
  if (s.workspace_bytes > kNoAllocScratchBytes) return TOPK_ERR_BUFFER_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != TOPK_OK) return st;
  // Clear what must start at zero on every call (the status word and the
  // split rows' group states; candidate slabs are written before they are
  // read): a previous call may have left them dirty by timing out, and every
  // call on this device shares them. A fill kernel, not a memset node.
  if (num_rows == 0) return TOPK_OK;
  const size_t clear = ws_cand_offset(s);
  if (launch_fill(ws, clear, (hipStream_t)stream) != hipSuccess) return TOPK_ERR_HIP;
  return select_impl(cfg, nullptr, scores, score_row_stride, lengths, num_rows, block_table, bt_row_stride,
                     page_size, out_slots, out_indices, out_row_stride, ws, s.workspace_bytes, stream, nullptr,
                     nullptr, device_status);
}

topk_status topk_debug_keys(const float* x, int64_t n, uint32_t* bin_out, uint32_t* key32_out, void* stream) {
  if (n < 0 || (n > 0 && !x)) return TOPK_ERR_INVALID_ARG;
  return launch_debug_keys(x, n, bin_out, key32_out, (hipStream_t)stream) == hipSuccess
             ? TOPK_OK
             : TOPK_ERR_HIP;
}

topk_status topk_debug_stream_read(const float* x, int64_t n, float* out, void* stream, void* start_event,
                                   void* stop_event) {
  if (n < 0 || (n > 0 && (!x || !out)) || ((uintptr_t)x % 16) != 0) return TOPK_ERR_INVALID_ARG;
  if (!start_event != !stop_event) return TOPK_ERR_INVALID_ARG;
  if (n / 4 == 0) return TOPK_OK;   // (a tail of fewer than 4 floats is not read)
  return launch_stream_read(x, n, out, (hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event) ==
                 hipSuccess
             ? TOPK_OK
             : TOPK_ERR_HIP;
}

int32_t topk_stream_read_groups(void) { return stream_read_groups(); }

topk_status topk_debug_histogram(const float* scores, int64_t score_row_stride, const int32_t* lengths,
                                 int32_t num_rows, int32_t k, uint32_t* hist_out, uint32_t* threshold_out,
                                 void* stream) {
  if (num_rows < 0 || k < 1 || k > kMaxK || score_row_stride < 0) return TOPK_ERR_INVALID_ARG;
  if (num_rows > 0 && (!scores || !lengths || !hist_out || !threshold_out)) return TOPK_ERR_INVALID_ARG;
  return launch_debug_hist(scores, score_row_stride, lengths, num_rows, k, hist_out, threshold_out,
                           (hipStream_t)stream) == hipSuccess
             ? TOPK_OK
             : TOPK_ERR_HIP;
}

const char* topk_status_string(topk_status s) {
  switch (s) {
    case TOPK_OK: return "ok";
    case TOPK_ERR_INVALID_ARG: return "invalid argument";
    case TOPK_ERR_BUFFER_TOO_SMALL: return "plan or workspace buffer too small";
    case TOPK_ERR_UNSUPPORTED: return "forced path cannot serve this configuration";
    case TOPK_ERR_HIP: return "HIP runtime error";
    case TOPK_ERR_DEVICE: return "device recorded an error";
  }
  return "unknown status";
}

}  // extern "C"
