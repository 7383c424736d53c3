// topk_layout.hpp -- tile sizes, plan and workspace layouts shared by the host
// launcher and the gfx950 kernels of the indexer top-k library.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace satopk {

// Workgroup shape: one 512-lane workgroup (8 wave64s) per CU, so it may use
// up to 256 VGPRs and most of the CU's 160 KB of LDS. Every lane holds kEpt
// scores of a register-resident tile as packed FP16 (kEpt / 4 dwordx4 loads
// in flight per lane, 128 KB per CU).
constexpr int kBlock = 512;
constexpr int kWave = 64;                // lanes per wavefront
constexpr int kWaves = kBlock / kWave;
constexpr int kEpt = 64;
constexpr int kTile = kBlock * kEpt;          // 32,768 scores = 128 KB per tile

constexpr int kMaxK = 2048;
constexpr int kBins = 1024;                   // top 10 bits of the 16-bit ordered key
constexpr int kRadixBits = 11;                // digit width of the exact refinement
constexpr int kRadixBins = 1 << kRadixBits;
constexpr int kListCap = 16384;               // boundary candidates kept in LDS (128 KB)
constexpr int kChunkAlign = 256;              // chunk starts are multiples of this
constexpr int kDefaultMinChunk = 4096;
constexpr int kDefaultCandCap = kListCap;     // boundary candidates per split row (fits the resolver's LDS)

constexpr uint32_t kPlanMagic = 0x31504B54u;  // "TKP1"
// Batches of at most this many rows are planned inside the selection kernel
// (one row per thread; every workgroup derives the same work list), so they
// need no planning launch and no plan buffer.
constexpr int kInKernelPlanRows = 512;
constexpr uint32_t kDefaultSpinLimit = 1u << 21;

// Plan buffer: header, then `capacity` work items.
struct PlanHeader {
  uint32_t magic;
  int32_t num_rows;
  int32_t num_items;        // items actually written
  int32_t num_multi_items;  // items [0, num_multi_items) belong to split rows
  int32_t grid;             // workgroups the selection launch uses
  int32_t k;
  int32_t num_groups;       // split rows (each owns one GroupState)
  int32_t chunk;            // planner's target chunk (diagnostic)
  int32_t pad[8];
};
static_assert(sizeof(PlanHeader) == 64, "plan header is 64 bytes");

struct WorkItem {
  int32_t row;
  int32_t begin;   // chunk [begin, end) of the row
  int32_t end;
  int32_t group;   // -1: the workgroup owns the whole row; else split-row slot
  int32_t gsize;   // workgroups sharing the row (1 for an owned row)
  int32_t len;     // the row's valid length as planned (-1: outside [0, max_len])
  int32_t pad[2];
};
static_assert(sizeof(WorkItem) == 32, "work item is 32 bytes");

// Boundary candidates of a split row are also counted by a 13-bit digit of
// their FP32 key, in a frame fixed by the threshold bin, so that the last
// workgroup starts its exact selection from a finished digit histogram.
constexpr int kFineBits = 13;
constexpr int kFineBins = 1 << kFineBits;
// The digits also add up in groups of 64 (coarse counts), which a reader
// polls instead of the whole digit histogram.
constexpr int kFineGroups = kFineBins / 64;

// Cross-workgroup state of one split row. Left zeroed after every use.
struct GroupState {
  uint32_t hist[kBins];   // merged 1,024-bin histogram
  // Added once per workgroup, each in one 64-bit atomic, so that the low
  // halves join the merged histogram's completeness check. High halves: the
  // workgroups that proposed a threshold bin (9 bits) and the sum of the
  // proposals (bin + 1) above them; the sum of the squared proposals.
  uint64_t arrive;        // low: scores of the row that no merged bin counts
  uint32_t emit;          // output cursor for scores above the threshold bin
  uint32_t cand;          // cursor into this row's candidate buffer
  uint32_t done;          // workgroups that finished emission
  uint32_t range[4];      // threshold-bin candidates: max key32, ~min key32, max pos, ~min pos
  uint32_t pad0[23];
  uint64_t vsq;           // low: workgroups; on a cache line of its own (atomics to one line queue)
  uint32_t pad1[30];
  uint32_t fine[kFineBins];   // threshold-bin candidates by FP32-key digit (large bins only)
  uint32_t fine_c[kFineGroups];   // the same by digit group, added once the group's digits have landed
};
static_assert(sizeof(GroupState) == 4096 + 256 + 4 * kFineBins + 4 * kFineGroups, "group state layout");
// Workgroups per split row stay below 2^9 (the proposer count's field).
constexpr int kMaxRowGroups = 511;

// The device status word sits at workspace offset 0.
constexpr size_t kStatusBytes = 256;

struct Sizing {
  int grid;          // persistent selection grid (<= co-resident capacity)
  int max_items;     // plan capacity in items
  int max_groups;    // split rows the workspace can hold
  int64_t cand_cap;  // candidates per split row
  size_t plan_bytes;
  size_t workspace_bytes;
};

// Workspace: [status, kStatusBytes][GroupState x max_groups][uint64 cand x max_groups x cand_cap]
inline size_t ws_group_offset() { return kStatusBytes; }
inline size_t ws_cand_offset(const Sizing& s) { return kStatusBytes + sizeof(GroupState) * (size_t)s.max_groups; }
inline size_t ws_total_bytes(const Sizing& s) {
  return ws_cand_offset(s) + sizeof(uint64_t) * (size_t)s.max_groups * (size_t)s.cand_cap;
}

struct PlanArgs {
  const int32_t* lengths;
  int32_t num_rows;
  int32_t k;
  int32_t grid;
  int32_t max_groups;
  int32_t max_items;
  int32_t force_path;
  int32_t wg_per_row;
  int32_t min_chunk;
  int64_t max_len;
  PlanHeader* header;
  WorkItem* items;
};

struct SelectArgs {
  const float* scores;
  int64_t stride;
  const int32_t* lengths;
  int32_t num_rows;
  int32_t k;
  const int32_t* table;
  int64_t table_stride;
  int32_t page_size;
  int32_t page_shift;     // log2(page_size) when a power of two, else -1
  int32_t* out_slots;
  int32_t* out_idx;       // may be null
  int64_t out_stride;
  const PlanHeader* plan;   // null: plan in the kernel (num_rows <= kInKernelPlanRows)
  const WorkItem* items;
  int32_t force_path;       // planning inputs, used when plan is null
  int32_t wg_per_row;
  int32_t min_chunk;
  int32_t max_groups;
  GroupState* groups;
  uint64_t* cand;
  int64_t cand_cap;
  int32_t* status;
  int64_t max_len;
  uint32_t spin_limit;
  int32_t guess_groups;     // in-kernel planning: the split of a max_len row when every
  int64_t guess_chunk;      // row has max_len scores (groups per row, chunk length)
};

}  // namespace satopk
