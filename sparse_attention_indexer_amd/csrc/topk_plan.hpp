// topk_plan.hpp -- the planner's rule for splitting rows across workgroups,
// shared by the planning kernel, the selection kernel's in-kernel planning
// and the host (which uses it to guess a batch's chunks before the lengths
// are read on the device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_topk.h"
#include "topk_layout.hpp"

namespace satopk {

// Quotient of non-negative integers below 2^52 from one correctly rounded
// FP64 division, corrected to the floor (the rounded quotient is within a
// quarter of the exact one, so it is the floor or one above it). A few
// instructions instead of the long emulated 64-bit integer division, which
// sits on the path to the first tile loads. Every operand here is below
// 2^52: lengths < 2^31, grids < 2^16, and a batch's total length is bounded
// by the scores it must fit in device memory.
__host__ __device__ __forceinline__ uint64_t udiv52(uint64_t a, uint64_t b) {
  uint64_t q = (uint64_t)((double)a / (double)b);
  if (q * b > a) --q;
  return q;
}
__host__ __device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) {
  return (int64_t)udiv52((uint64_t)(a + b - 1), (uint64_t)b);
}
__host__ __device__ __forceinline__ int64_t round_up64(int64_t a, int64_t b) { return ceil_div64(a, b) * b; }

// Workgroups a row of `len` scores gets (1 = the row stays whole).
//  - fixed: a fixed group size for every row longer than k;
//  - force_split: at least 2, the grid's remaining workgroups shared in
//    proportion to length (at most 2 per row + the rest: fits one round);
//  - otherwise: rows that fit one register tile stay whole; each takes one
//    item, and the rest of the grid (the budget) goes to the longer rows.
//    A longer row first gets one workgroup per register tile it spans (so
//    every chunk stays register-resident), when those add up to no more than
//    the budget (`tiles` is their sum over the batch); the rest of the budget
//    is shared in proportion to length, floor-rounded, so all items fit one
//    round of the persistent grid, with no chunk shorter than min_chunk.
// `total` and `n_long` sum over the rows this mode splits: longer than one
// tile by default, longer than k under a forced split or fixed group size.
// The chunk is then aligned to kChunkAlign, which can only lower the count.
__host__ __device__ __forceinline__ int64_t tiles_of(int32_t len) { return len > kTile ? ceil_div64(len, kTile) : 0; }
__host__ __device__ __forceinline__ int32_t split_floor(const PlanArgs& a) {
  return (a.force_path == TOPK_PATH_AUTO && a.wg_per_row <= 0) ? (kTile > a.k ? kTile : a.k) : a.k;
}

__host__ __device__ __forceinline__ int split_of(int32_t len, const PlanArgs& a, uint64_t total, int32_t n_long,
                                        uint32_t tiles, int64_t* chunk_out) {
  *chunk_out = len;
  if (len <= a.k || total == 0) return 1;
  int64_t g;
  if (a.wg_per_row > 0) {
    g = a.wg_per_row;
  } else if (a.force_path == TOPK_PATH_MULTI) {
    const int64_t spare = (int64_t)a.grid - 2 * (int64_t)n_long;
    g = 2 + (spare > 0 ? (int64_t)udiv52((uint64_t)spare * (uint64_t)len, total) : 0);
  } else if (a.force_path == TOPK_PATH_REGISTER || a.force_path == TOPK_PATH_SINGLE) {
    return 1;
  } else {
    // A row that fits one workgroup's register tile stays whole: one pass
    // with no cross-workgroup exchange beats any split of it.
    if (len <= kTile) return 1;
    const int64_t budget = (int64_t)a.grid - ((int64_t)a.num_rows - n_long);
    if (budget >= (int64_t)tiles)
      g = tiles_of(len) + (int64_t)udiv52((uint64_t)(budget - (int64_t)tiles) * (uint64_t)len, total);
    else
      g = (int64_t)udiv52((uint64_t)a.grid * (uint64_t)len, total);
    const int64_t min_chunk = a.min_chunk > 0 ? a.min_chunk : kDefaultMinChunk;
    const int64_t by_min = (int64_t)udiv52((uint64_t)len, (uint64_t)min_chunk);
    if (g > by_min) g = by_min;
  }
  if (g < 2) return 1;
  const int64_t c = round_up64(ceil_div64(len, g), kChunkAlign);
  g = ceil_div64(len, c);
  if (g < 2) return 1;
  *chunk_out = c;
  return (int)g;
}

}  // namespace satopk
