// topk_kernels.hip -- gfx950 kernels of the indexer top-k library.
//
// The method follows the TopK-V2 section of the lmsys.org page "Serving GLM5.2
// NVFP4 Agentic Workload with SGLang" (text and Figures 2-4): top-k is treated
// as selection, not sorting. Each score is rounded to FP16 and binned by the
// top 10 bits of an order-preserving key (1,024 bins); the bin holding the
// k-th largest score is located from the histogram; scores in higher bins are
// emitted directly; scores in the boundary bin are resolved by an exact radix
// selection on their FP32 keys with a position tie-break; every selected
// position is mapped through the paged block table in the same kernel. A
// planning kernel picks, per row, how many workgroups share it and writes a
// work list that the selection kernel's persistent grid consumes.
//
// Differences from the page's Blackwell design (which uses 8-CTA thread-block
// clusters and a cluster-wide reduction): gfx950 has no clusters, so the
// workgroups that split a long row merge their histograms with device-scope
// atomics into a per-row global histogram and meet at a bounded spin barrier;
// the last workgroup to finish emission resolves the boundary bin from a
// global candidate buffer. Workgroups of a split row only merge bins at or
// above their own local k-th bin, since the row's k-th score can never lie
// below any chunk's k-th score.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "sparse_topk.h"
#include "topk_device.hpp"
#include "topk_layout.hpp"
#include "topk_plan.hpp"

namespace satopk {

// ---------------------------------------------------------------------------
// Planning kernel: one workgroup reads the device lengths and writes the plan.
// ---------------------------------------------------------------------------
constexpr int kPlanBlock = 256;

constexpr int kPlanWaves = kPlanBlock / 64;

__global__ void __launch_bounds__(kPlanBlock) topk_plan_kernel(PlanArgs a) {
  __shared__ uint64_t s_red[kPlanWaves];
  __shared__ uint64_t s_red2[kPlanWaves];
  __shared__ uint32_t s_scan[kPlanWaves];
  __shared__ int s_carry_multi, s_carry_groups, s_carry_single;
  const int t = threadIdx.x;

  // Total length and count of the rows longer than k (wave sums, then one
  // LDS word per wave: no same-address atomics).
  uint64_t mine = 0;
  uint32_t longs = 0;
  uint64_t tl = 0;
  const int32_t floor_len = split_floor(a);
  for (int r = t; r < a.num_rows; r += kPlanBlock) {
    const int32_t len = a.lengths[r];
    if (len > floor_len) {
      mine += (uint64_t)len;
      ++longs;
      tl += (uint64_t)tiles_of(len);
    }
  }
  mine = wave_sum_u64(mine + ((uint64_t)longs << 40));   // lengths < 2^31, rows < 2^23
  tl = wave_sum_u64(tl);
  if (lane() == 0) {
    s_red[t >> 6] = mine;
    s_red2[t >> 6] = tl;
  }
  __syncthreads();
  uint64_t packed = 0, tiles64 = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    packed += s_red[i];
    tiles64 += s_red2[i];
  }
  const uint32_t tiles = (uint32_t)min(tiles64, (uint64_t)0xFFFFFFFFu);   // saturated: > grid either way
  const uint64_t total = packed & ((1ull << 40) - 1);
  const int32_t n_long = (int32_t)(packed >> 40);
  if (t == 0) {
    s_carry_multi = 0;
    s_carry_groups = 0;
    s_carry_single = 0;
  }
  __syncthreads();

  // Items: split rows first (indices [0, total_multi), one grid round), then
  // one item per whole row. Three scans over each block of rows.
  // First count the split rows' items so whole rows can start after them.
  uint32_t my_multi = 0, my_groups = 0;
  for (int r = t; r < a.num_rows; r += kPlanBlock) {
    int64_t c;
    const int g = split_of(a.lengths[r], a, total, n_long, tiles, &c);
    if (g > 1) {
      my_multi += (uint32_t)g;
      my_groups += 1;
    }
  }
  uint32_t total_multi_u, total_groups_u;
  block_exclusive_add<kPlanWaves>(my_multi, s_scan, &total_multi_u);
  block_exclusive_add<kPlanWaves>(my_groups, s_scan, &total_groups_u);
  const int total_multi = (int)total_multi_u;
  if (total_multi > a.grid || (int)total_groups_u > a.max_groups) {
    // unreachable for configurations the host accepts; never hand out a
    // plan whose split rows cannot all be resident at once
    if (t == 0) {
      a.header->magic = 0;
      a.header->num_items = 0;
    }
    return;
  }
  for (int r0 = 0; r0 < a.num_rows; r0 += kPlanBlock) {
    const int r = r0 + t;
    int g = 0;
    int64_t c = 0;
    int32_t len = 0;
    if (r < a.num_rows) {
      len = a.lengths[r];
      g = split_of(len, a, total, n_long, tiles, &c);
    }
    const uint32_t n_multi = (r < a.num_rows && g > 1) ? (uint32_t)g : 0u;
    const uint32_t n_group = n_multi ? 1u : 0u;
    const uint32_t n_single = (r < a.num_rows && g == 1) ? 1u : 0u;
    uint32_t tot_m, tot_g, tot_s;
    const uint32_t off_m = block_exclusive_add<kPlanWaves>(n_multi, s_scan, &tot_m);
    const uint32_t off_g = block_exclusive_add<kPlanWaves>(n_group, s_scan, &tot_g);
    const uint32_t off_s = block_exclusive_add<kPlanWaves>(n_single, s_scan, &tot_s);
    const int base_m = s_carry_multi, base_g = s_carry_groups, base_s = s_carry_single;
    if (n_multi) {
      const int first = base_m + (int)off_m;
      const int gid = base_g + (int)off_g;
      for (int j = 0; j < g; ++j) {
        WorkItem w;
        w.row = r;
        w.begin = (int32_t)(j * c);
        const int64_t e = (int64_t)(j + 1) * c;
        w.end = (int32_t)(e < len ? e : len);
        w.group = gid;
        w.gsize = g;
        w.len = len;
        w.pad[0] = w.pad[1] = 0;
        a.items[first + j] = w;
      }
    }
    if (n_single) {
      WorkItem w;
      w.row = r;
      w.begin = 0;
      w.end = len;
      w.group = -1;
      w.gsize = 1;
      w.len = (len < 0 || (int64_t)len > a.max_len) ? -1 : len;
      w.pad[0] = w.pad[1] = 0;
      a.items[total_multi + base_s + (int)off_s] = w;
    }
    __syncthreads();
    if (t == 0) {
      s_carry_multi += (int)tot_m;
      s_carry_groups += (int)tot_g;
      s_carry_single += (int)tot_s;
    }
    __syncthreads();
  }
  if (t == 0) {
    PlanHeader h;
    h.magic = kPlanMagic;
    h.num_rows = a.num_rows;
    h.num_items = total_multi + s_carry_single;
    h.num_multi_items = total_multi;
    h.grid = a.grid;
    h.k = a.k;
    h.num_groups = s_carry_groups;
    const uint64_t even = total / (uint64_t)(a.grid > 0 ? a.grid : 1);
    h.chunk = (int32_t)(even > 0x7FFFFFFFull ? 0x7FFFFFFFull : even);
    for (int i = 0; i < 8; ++i) h.pad[i] = 0;
    *a.header = h;
  }
}

// ---------------------------------------------------------------------------
// Selection kernel
// ---------------------------------------------------------------------------
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Two scores -> two FP16 values (round to nearest even) in one register, then
// +0 is added so that -0 becomes +0 and equal scores share a bin.
__device__ __forceinline__ uint32_t to_half2(float a, float b) {
  half2v v;
  v.x = (_Float16)a;
  v.y = (_Float16)b;
  v = v + (half2v){(_Float16)0.0f, (_Float16)0.0f};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ _Float16 half_lo(uint32_t p) { return __builtin_bit_cast(half2v, p).x; }
__device__ __forceinline__ _Float16 half_hi(uint32_t p) { return __builtin_bit_cast(half2v, p).y; }
__device__ __forceinline__ _Float16 half_of_bits(uint32_t b) { return __builtin_bit_cast(_Float16, (uint16_t)b); }

// Registers of positions past the chunk end hold this quiet NaN: it never
// compares >= anything and its histogram bin (key bin 1016) is never scanned.
constexpr uint32_t kHalfNaN = 0x7E00u;
constexpr uint32_t kHalfNaN2 = 0x7E007E00u;

// The LDS histogram is indexed by the raw top 10 bits of the canonical FP16
// value (sign, exponent, 4 mantissa bits). Ordered-key bin b lives at raw
// index raw_of_bin(b): non-negative values keep their order, negative ones
// reverse it. Key bins 0..14 and 1009..1023 hold only NaN codes.
__device__ __forceinline__ uint32_t raw_of_bin(uint32_t b) { return b >= 512u ? b - 512u : 1023u - b; }
__device__ __forceinline__ uint32_t bin_of_raw(uint32_t r) { return r < 512u ? r + 512u : 1023u - r; }
constexpr uint32_t kFirstBin = 15, kLastBin = 1008;   // -inf bin, +inf bin
constexpr uint32_t kNotFound = 0xFFFFFFFFu;

// For threshold bin b*: bin(x) >= b* <=> h >= vlo and bin(x) > b* <=> h >= vhi,
// with h the canonical FP16 of x (FP16 order agrees with key order off -0/NaN;
// FP16 denormals are kept, so the comparison is exact).
struct Cut {
  _Float16 vlo, vhi;
};
__device__ __forceinline__ uint32_t half_bits_of_key16(uint32_t key) {
  return (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
}
__device__ __forceinline__ Cut cut_of_bin(uint32_t b) {
  const uint32_t tlo = b * 64u, thi = (b + 1u) * 64u;
  Cut c;
  c.vlo = half_of_bits(tlo >= 0x03FFu ? half_bits_of_key16(tlo) : 0xFC00u);     // at most -inf
  c.vhi = half_of_bits(thi <= 0xFC00u ? half_bits_of_key16(thi) : kHalfNaN);    // NaN: none above
  return c;
}

// Cross-workgroup traffic goes through device-coherent operations only:
// atomics, and loads/stores at agent scope (which bypass the non-coherent
// per-XCD L2). Each wave drains its own memory operations before the
// workgroup barrier that precedes an arrival count, so no whole-cache
// writeback or invalidate (an agent-scope fence) is ever needed.
__device__ __forceinline__ void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }
template <class T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kFirstRadixBits = 13;                 // first refinement digit (histogram in the list region)
constexpr int kFirstRadixBins = 1 << kFirstRadixBits;
constexpr int kWidePad = 4;                         // one pad word per 16 bins: conflict-free threshold scan
constexpr int kWideWords = kFirstRadixBins + (kFirstRadixBins >> kWidePad);
constexpr int kWideSlots = kWideWords / 2;          // list entries the padded histogram occupies
constexpr int kResolveRegs = 24;                    // candidates per lane of the register-resident first pass
// While a split row's workgroup waits for the others it re-reads the scores
// that will probably be needed: those in bins at or above the one holding
// its own T-th largest score, T = 2 * ceil(k / G) + 64 (twice its share of
// the row's top k when scores are spread evenly). If the row's threshold bin
// turns out lower, the workgroup re-reads from the tile instead. Up to
// kPreRegs per lane; positions are listed in the top of the LDS list, values
// and block-table entries held in registers.
constexpr int kPreRegs = 4;
constexpr int kPreCap = kPreRegs * kBlock;
constexpr int kStageCap = kListCap - kPreCap / 2;  // staged candidates below the position list
// A split row's per-workgroup fine-digit counters (32 KB) sit in the LDS list
// above at most kFineListOff staged candidates and below the position list.
constexpr int kFineListOff = 8192;
static_assert(kFineListOff + kFineBins / 2 <= kStageCap, "fine-digit counters below the position list");
// The per-workgroup digit-group sums (128 words) follow the digit counters.
constexpr int kFineGroupOff = kFineListOff + kFineBins / 2;   // (list entries)
// A workgroup that classifies its chunk before the row's histogram is merged
// (a predicted crowded threshold bin, see split_row) stages its outputs above
// that bin (positions, then block-table entries) here, clear of the merged
// histogram it is about to read into rhist and of the prefixes in outpos.
constexpr int kSpecStageOff = kFineGroupOff + kFineGroups / 2;
static_assert(kSpecStageOff + kMaxK <= kStageCap, "predicted-bin outputs below the position list");
static_assert(kWideWords * 4 <= kListCap * 8, "first-digit histogram aliases the LDS list");
static_assert(kMaxK <= kRadixBins, "above-threshold staging aliases rhist");

// Items one workgroup takes from an in-kernel plan: at most one split item
// (split rows fit one grid round) plus ceil(rows / grid) whole rows.
constexpr int kMaxLocalItems = 16;

struct __align__(16) Smem {
  uint64_t list[kListCap];      // boundary candidates: (key32 << 32 | position), then composite keys
  uint32_t lhist[kBins];        // this workgroup's histogram (raw index)
  uint32_t rhist[kRadixBins];   // refinement digits; merged histogram; staged above-threshold positions
  uint32_t outpos[kMaxK];       // a row's selected positions, by output index, until the flush
  uint32_t scratch[kWaves];
  uint32_t res[4];
  uint32_t cur_out;             // next output position of the row
  uint32_t cur_list;            // next candidate position (LDS list or global buffer)
  uint32_t flag;
  uint32_t range[4];            // candidate key/position range: kmax, ~kmin, imax, ~imin
  uint32_t bcast[4];
  uint64_t pl_red[kWaves];
  uint32_t pl_red2[kWaves];
  WorkItem pl_items[kMaxLocalItems];   // in-kernel plan: this workgroup's items, in loop order
};

// Output of one row: slot = table[i / ps] * ps + i % ps (page: TopK-V2,
// selected logical positions translated to physical indexer KV-cache slots).
// write() stages a position in LDS; flush() then maps and stores a range of
// outputs with all block-table loads in flight at once. Every write checks
// its bounds and returns false instead of writing out of range; callers
// gather the flags and report them once (report_bad).
struct RowOut {
  int32_t* slots;
  int32_t* idx;
  const int32_t* table;
  int32_t ps;
  int32_t shift;
  uint32_t k;
  uint32_t len;      // valid positions of the row
  int32_t* status;
  uint32_t* stage;   // LDS, k entries

  __device__ __forceinline__ bool write(uint32_t pos, int32_t i) const {
    const bool ok = pos < k;
    if (ok) stage[pos] = (uint32_t)i;
    return ok;
  }

  __device__ __forceinline__ int32_t page(int32_t i) const {
    return shift >= 0 ? table[i >> shift] : table[i / ps];
  }

  // Output pos <- position i whose block-table entry `pg` is already known.
  __device__ __forceinline__ bool store_page(uint32_t pos, int32_t i, int32_t pg) const {
    const bool ok = pos < k && (uint32_t)i < len;
    if (ok) {
      slots[pos] = pg * ps + (shift >= 0 ? (i & (ps - 1)) : (i % ps));
      if (idx) idx[pos] = i;
    }
    return ok;
  }

  __device__ __forceinline__ bool store(uint32_t pos, int32_t i) const {
    const bool ok = pos < k && (uint32_t)i < len;   // never index the table past the row
    return ok ? store_page(pos, i, page(i)) : false;
  }

  // Whole workgroup; staged outputs [from, to), to <= k <= kMaxK. Each lane
  // takes up to kFlushPer outputs and has all their block-table loads in
  // flight before the first store (one round trip rather than one per
  // output).
  static constexpr int kFlushPer = kMaxK / kBlock;
  static_assert(kFlushPer * kBlock == kMaxK, "the lanes' flush slots cover k");
  __device__ __forceinline__ bool flush(uint32_t from, uint32_t to) const {
    bool ok = true;
    int32_t e[kFlushPer], pg[kFlushPer];
    bool v[kFlushPer];
#pragma unroll
    for (int u = 0; u < kFlushPer; ++u) {
      const uint32_t j = from + threadIdx.x + (uint32_t)u * kBlock;
      v[u] = j < to;
      e[u] = v[u] ? (int32_t)stage[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < kFlushPer; ++u)   // never index the table past the row
      pg[u] = (v[u] && (uint32_t)e[u] < len) ? page(e[u]) : 0;
#pragma unroll
    for (int u = 0; u < kFlushPer; ++u)
      if (v[u]) ok &= store_page(from + threadIdx.x + (uint32_t)u * kBlock, e[u], pg[u]);
    return ok;
  }
};

// One device-status flag for every lane that saw an inconsistency (counts and
// classification disagreeing, which valid inputs never cause). Whole wave.
__device__ __forceinline__ void report_bad(bool bad, int32_t* status) {
  if (__ballot(bad) != 0ull && lane() == 0) atomicOr(status, TOPK_DEVICE_INTERNAL);
}

// Wave-aggregated output: one LDS atomic per wave reserves positions.
__device__ __forceinline__ bool emit_wave(bool take, int32_t i, uint32_t* cursor, const RowOut& o) {
  const uint64_t m = __ballot(take);
  if (m == 0) return true;
  const uint32_t leader = first_lane(m);
  uint32_t base = 0;
  if (lane() == leader) base = atomicAdd(cursor, (uint32_t)__popcll(m));
  base = read_lane(base, leader);
  return take ? o.write(base + mbcnt(m), i) : true;
}

__device__ __forceinline__ void push_wave(bool take, uint64_t v, uint32_t* cursor, uint64_t* dst) {
  const uint64_t m = __ballot(take);
  if (m == 0) return;
  const uint32_t leader = first_lane(m);
  uint32_t base = 0;
  if (lane() == leader) base = atomicAdd(cursor, (uint32_t)__popcll(m));
  base = read_lane(base, leader);
  if (take) dst[base + mbcnt(m)] = v;
}

// Element j = q * 4 + c of a lane's tile sits at this position: lane t loads
// dwordx4 number q at (q * kBlock + t) * 4, so each load instruction of a wave
// reads 1 KB of consecutive scores. Packed register hk[j / 2] holds elements
// j & ~1 (low half) and j | 1 (high half).
__device__ __forceinline__ int32_t tile_pos(int32_t base, int q, int c) {
  return base + (q * kBlock + (int)threadIdx.x) * 4 + c;
}

constexpr int kHk = kEpt / 2;   // packed registers per lane

// A tile's raw dwordx4 loads: lane t's vector q holds positions
// tile_pos(base, q, 0..3); vectors that start at or past `end` are not read.
template <bool VEC>
__device__ __forceinline__ void load_raw(const float* rowp, int32_t base, int32_t end, float4 (&x)[kEpt / 4]) {
#pragma unroll
  for (int q = 0; q < kEpt / 4; ++q) {
    const int32_t e = tile_pos(base, q, 0);
    x[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (VEC) {
      // Rows are 16-byte aligned and their stride is a multiple of 4, so a
      // vector that starts before `end` lies inside the row.
      if (e < end) x[q] = *reinterpret_cast<const float4*>(rowp + e);
    } else {
      if (e < end) x[q].x = rowp[e];
      if (e + 1 < end) x[q].y = rowp[e + 1];
      if (e + 2 < end) x[q].z = rowp[e + 2];
      if (e + 3 < end) x[q].w = rowp[e + 3];
    }
  }
}

// The same loads through a buffer resource that covers [base, end) of the
// row (at most one tile): positions at or past `end` read as zero without a
// memory access and without a branch, so every load is issued
// unconditionally. (A load under a per-lane branch lets the compiler move
// its first use into the branch, where the wait for it also waits for every
// earlier load; the speculative tile load must not wait before the planning
// that overlaps it.) Consumers mask positions past `end` as for load_raw.
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

// Only the first NV vector groups are read; the others hold zeros (the
// caller guarantees [base, end) lies within them).
template <bool VEC, int NV = kEpt / 4>
__device__ __forceinline__ void load_raw_buffer(const float* rowp, int32_t base, int32_t end,
                                                float4 (&x)[kEpt / 4]) {
  const int32_t n = end > base ? min(end - base, (int32_t)kTile) : 0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(rowp) + base, (short)0, n * 4, kBufferFlags);
#pragma unroll
  for (int q = NV; q < kEpt / 4; ++q) x[q] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int32_t off = (q * kBlock + (int)threadIdx.x) * 16;   // bytes from `base`
    if constexpr (VEC) {
      x[q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    } else {
      x[q].x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
      x[q].y = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4, 0, 0));
      x[q].z = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + 8, 0, 0));
      x[q].w = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + 12, 0, 0));
    }
  }
}

// Raw loads -> packed FP16 tile; positions at or past `end` become NaN.
__device__ __forceinline__ void pack_tile(const float4 (&x)[kEpt / 4], int32_t base, int32_t end,
                                          uint32_t (&hk)[kHk]) {
#pragma unroll
  for (int q = 0; q < kEpt / 4; ++q) {
    const int32_t e = tile_pos(base, q, 0);
    uint32_t p0 = to_half2(x[q].x, x[q].y), p1 = to_half2(x[q].z, x[q].w);
    if (e + 4 > end) {  // tail vector: positions >= end become NaN
      const int n = end - e;
      p0 = n <= 0 ? kHalfNaN2 : (n == 1 ? (p0 & 0xFFFFu) | (kHalfNaN << 16) : p0);
      p1 = n <= 2 ? kHalfNaN2 : (n == 3 ? (p1 & 0xFFFFu) | (kHalfNaN << 16) : p1);
    }
    hk[2 * q] = p0;
    hk[2 * q + 1] = p1;
  }
}

template <bool VEC>
__device__ __forceinline__ void load_pack(const float* rowp, int32_t base, int32_t end, uint32_t (&hk)[kHk]) {
  float4 x[kEpt / 4];
  load_raw<VEC>(rowp, base, end, x);
  pack_tile(x, base, end, hk);
}

// Histograms of a tile go into kHistCopies interleaved copies of the
// 1,024 counters (bin r, copy c at word r * kHistCopies + c; lane l adds to
// copy l % kHistCopies), so lanes that hit one hot bin in the same
// instruction mostly land on different words and banks. When one bin takes
// all 256 scores of a wave's dwordx4 (all-equal or one-bin rows), a single
// atomic adds 256. NaN padding lands in an unscanned bin; dwordx4 groups
// wholly past `end` are skipped (the test is uniform across the workgroup).
constexpr int kHistCopies = 8;   // (16 measured slower: more LDS to clear and sum)
static_assert(kBins * kHistCopies * 4 <= kListCap * 8, "histogram copies fit in the LDS list region");

// Pack a tile (as pack_tile) and bin it into the copies in one pass over the
// vectors, in load order, so the atomics of vector q go out while later
// vectors are still arriving.
template <int NQ = kEpt / 4>
__device__ __forceinline__ void pack_hist(const float4 (&x)[kEpt / 4], int32_t base, int32_t end,
                                          uint32_t (&hk)[kHk], uint32_t* hc) {
  const uint32_t c = threadIdx.x & (kHistCopies - 1);
  // NQ < kEpt / 4: the caller guarantees end <= base + NQ * kBlock * 4, so
  // the later vector groups hold no position below `end` (NaN throughout).
#pragma unroll
  for (int q = NQ; q < kEpt / 4; ++q) hk[2 * q] = hk[2 * q + 1] = kHalfNaN2;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int32_t e = tile_pos(base, q, 0);
    uint32_t p0 = to_half2(x[q].x, x[q].y), p1 = to_half2(x[q].z, x[q].w);
    if (e + 4 > end) {  // tail vector: positions >= end become NaN
      const int n = end - e;
      p0 = n <= 0 ? kHalfNaN2 : (n == 1 ? (p0 & 0xFFFFu) | (kHalfNaN << 16) : p0);
      p1 = n <= 2 ? kHalfNaN2 : (n == 3 ? (p1 & 0xFFFFu) | (kHalfNaN << 16) : p1);
    }
    hk[2 * q] = p0;
    hk[2 * q + 1] = p1;
    if (base + q * kBlock * 4 < end) {   // uniform
      const uint32_t r0 = (p0 >> 6) & 0x3FFu, r1 = p0 >> 22, r2 = (p1 >> 6) & 0x3FFu, r3 = p1 >> 22;
      const uint32_t f = (uint32_t)__builtin_amdgcn_readfirstlane((int)r0);
      const bool same = r0 == f && r1 == f && r2 == f && r3 == f;
      if (__ballot(same) == ~0ull) {
        if (lane() == 0) atomicAdd(&hc[f * kHistCopies + c], 256u);
      } else {
        atomicAdd(&hc[r0 * kHistCopies + c], 1u);
        atomicAdd(&hc[r1 * kHistCopies + c], 1u);
        atomicAdd(&hc[r2 * kHistCopies + c], 1u);
        atomicAdd(&hc[r3 * kHistCopies + c], 1u);
      }
    }
  }
}

// N dwordx4 per lane at positions base + (u * kBlock + t) * 4 (vectors that
// start at or past `end` are not read), and their histogram (same layout and
// fast path as pack_hist; positions past `end` are NaN).
template <bool VEC, int N>
__device__ __forceinline__ void load_vecs(const float* rowp, int32_t base, int32_t end, float4 (&x)[N]) {
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int32_t e = base + (u * kBlock + (int)threadIdx.x) * 4;
    x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (VEC) {
      if (e < end) x[u] = *reinterpret_cast<const float4*>(rowp + e);
    } else {
      if (e < end) x[u].x = rowp[e];
      if (e + 1 < end) x[u].y = rowp[e + 1];
      if (e + 2 < end) x[u].z = rowp[e + 2];
      if (e + 3 < end) x[u].w = rowp[e + 3];
    }
  }
}

template <int N>
__device__ __forceinline__ void hist_vecs(const float4 (&x)[N], uint32_t* hc, int32_t base, int32_t end) {
  const uint32_t c = threadIdx.x & (kHistCopies - 1);
#pragma unroll
  for (int u = 0; u < N; ++u) {
    if (base + u * kBlock * 4 >= end) break;
    const int32_t e = base + (u * kBlock + (int)threadIdx.x) * 4;
    uint32_t p0 = to_half2(x[u].x, x[u].y), p1 = to_half2(x[u].z, x[u].w);
    if (e + 4 > end) {
      const int n = end - e;
      p0 = n <= 0 ? kHalfNaN2 : (n == 1 ? (p0 & 0xFFFFu) | (kHalfNaN << 16) : p0);
      p1 = n <= 2 ? kHalfNaN2 : (n == 3 ? (p1 & 0xFFFFu) | (kHalfNaN << 16) : p1);
    }
    const uint32_t r0 = (p0 >> 6) & 0x3FFu, r1 = p0 >> 22, r2 = (p1 >> 6) & 0x3FFu, r3 = p1 >> 22;
    const uint32_t f = (uint32_t)__builtin_amdgcn_readfirstlane((int)r0);
    const bool same = r0 == f && r1 == f && r2 == f && r3 == f;
    if (__ballot(same) == ~0ull) {
      if (lane() == 0) atomicAdd(&hc[f * kHistCopies + c], 256u);
    } else {
      atomicAdd(&hc[r0 * kHistCopies + c], 1u);
      atomicAdd(&hc[r1 * kHistCopies + c], 1u);
      atomicAdd(&hc[r2 * kHistCopies + c], 1u);
      atomicAdd(&hc[r3 * kHistCopies + c], 1u);
    }
  }
}

// Zero the histogram copies (whole workgroup; a barrier must follow).
__device__ __forceinline__ void hist_copies_clear(uint32_t* hc) {
  uint4* p = reinterpret_cast<uint4*>(hc);
  for (int i = threadIdx.x; i < kBins * kHistCopies / 4; i += kBlock) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Sum the copies into h[0, kBins) (whole workgroup; a barrier must follow).
__device__ __forceinline__ void hist_copies_sum(const uint32_t* hc, uint32_t* h) {
  for (int r = threadIdx.x; r < kBins; r += kBlock) {
    const uint4* p = reinterpret_cast<const uint4*>(hc + r * kHistCopies);
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kHistCopies / 4; ++i) {
      const uint4 v = p[i];
      sum += v.x + v.y + v.z + v.w;
    }
    h[r] = sum;
  }
}

// Bit j set <=> element j lies in the threshold bin or above it. The words
// are shifted in from the top element down, (m << 1) | bit: setting bit j
// directly would need the constant 1 << j in a register for every j above
// 6 (these instructions take no 32-bit literal), and the compiler keeps
// such constants in registers for the whole kernel.
__device__ __forceinline__ uint64_t interest_mask(const uint32_t (&hk)[kHk], _Float16 vlo) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = kHk / 2 - 1; i >= 0; --i) {
    lo = (lo << 1) | (uint32_t)(half_hi(hk[i]) >= vlo);
    lo = (lo << 1) | (uint32_t)(half_lo(hk[i]) >= vlo);
    hi = (hi << 1) | (uint32_t)(half_hi(hk[i + kHk / 2]) >= vlo);
    hi = (hi << 1) | (uint32_t)(half_lo(hk[i + kHk / 2]) >= vlo);
  }
  return ((uint64_t)hi << 32) | lo;
}
static_assert(kEpt == 64, "interest_mask packs one bit per tile element into 64 bits");

// Per-lane running range of the boundary candidates, all kept as maxima.
struct Range {
  uint32_t kmax = 0, kmin_inv = 0, imax = 0, imin_inv = 0;
};

// Re-reads go out kReload at a time so their latencies overlap. With a table,
// each position's block-table entry is fetched in the same round trip and
// handed to on_above, so staged outputs need no second lookup.
constexpr int kReload = 4;

// The few positions of `mask` are re-read as FP32 and classified: above the
// threshold bin -> on_above(position); in it -> counted into the range and
// passed to on_cand(key32, position).
template <class A, class C>
__device__ __forceinline__ void extract(uint64_t mask, int32_t base, const float* rowp, _Float16 vhi, Range& rg,
                                        A&& on_above, C&& on_cand, const RowOut* pages = nullptr) {
  while (mask) {
    int32_t e[kReload];
    bool v[kReload];
#pragma unroll
    for (int u = 0; u < kReload; ++u) {
      v[u] = mask != 0ull;
      const int j = v[u] ? __builtin_ctzll(mask) : 0;
      mask &= mask - 1ull;
      e[u] = tile_pos(base, j >> 2, j & 3);
    }
    float x[kReload];
    int32_t pg[kReload];
#pragma unroll
    for (int u = 0; u < kReload; ++u) {
      x[u] = v[u] ? rowp[e[u]] : 0.f;
      pg[u] = (v[u] && pages) ? pages->page(e[u]) : 0;
    }
#pragma unroll
    for (int u = 0; u < kReload; ++u) {
      if (!v[u]) continue;
      if (half_lo(to_half2(x[u], x[u])) >= vhi) {
        on_above(e[u], pg[u]);
      } else {
        const uint32_t kk = key32_of(x[u]);
        rg.kmax = max(rg.kmax, kk);
        rg.kmin_inv = max(rg.kmin_inv, ~kk);
        rg.imax = max(rg.imax, (uint32_t)e[u]);
        rg.imin_inv = max(rg.imin_inv, ~(uint32_t)e[u]);
        on_cand(kk, e[u]);
      }
    }
  }
}

// One position whose FP32 score x may lie at or above the threshold bin:
// above it -> on_above(position, page); in it -> range and on_cand.
template <class A, class C>
__device__ __forceinline__ void classify(float x, int32_t e, int32_t pg, Cut cut, Range& rg, A&& on_above,
                                         C&& on_cand) {
  const _Float16 h = half_lo(to_half2(x, x));
  if (h >= cut.vhi) {
    on_above(e, pg);
  } else if (h >= cut.vlo) {
    const uint32_t kk = key32_of(x);
    rg.kmax = max(rg.kmax, kk);
    rg.kmin_inv = max(rg.kmin_inv, ~kk);
    rg.imax = max(rg.imax, (uint32_t)e);
    rg.imin_inv = max(rg.imin_inv, ~(uint32_t)e);
    on_cand(kk, e);
  }
}

// Merge the lanes' ranges into sh.range (LDS, zeroed beforehand).
__device__ __forceinline__ void merge_range(Range rg, Smem& sh) {
  rg.kmax = wave_max(rg.kmax);
  rg.kmin_inv = wave_max(rg.kmin_inv);
  rg.imax = wave_max(rg.imax);
  rg.imin_inv = wave_max(rg.imin_inv);
  if (lane() == 0) {
    atomicMax(&sh.range[0], rg.kmax);
    atomicMax(&sh.range[1], rg.kmin_inv);
    atomicMax(&sh.range[2], rg.imax);
    atomicMax(&sh.range[3], rg.imin_inv);
  }
}

// Scan the 1,024 ordered bins from the top (through raw_of_bin) and find the
// one holding the need-th largest score. NaN-only bins count as empty.
__device__ __forceinline__ void find_threshold_raw(const uint32_t* hist, uint32_t need, uint32_t* scratch,
                                                   uint32_t* result) {
  constexpr int PB = kBins / kBlock;
  const int t = threadIdx.x;
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const uint32_t b = (uint32_t)(kBins - 1 - (t * PB + j));
    s += (b >= kFirstBin && b <= kLastBin) ? hist[raw_of_bin(b)] : 0u;
  }
  uint32_t cum = block_exclusive_add(s, scratch);
  if (cum < need && need <= cum + s) {
    for (int j = 0; j < PB; ++j) {
      const uint32_t b = (uint32_t)(kBins - 1 - (t * PB + j));
      const uint32_t h = (b >= kFirstBin && b <= kLastBin) ? hist[raw_of_bin(b)] : 0u;
      if (cum < need && need <= cum + h) {
        result[0] = b;
        result[1] = cum;
        result[2] = h;
        break;
      }
      cum += h;
    }
  }
  __syncthreads();
}

// One scan of a chunk's histogram from the top (as find_threshold_raw) that
// finds two thresholds at once, the bins holding the need1-th and need2-th
// largest scores (*b1, *b2: left as preset when the chunk holds fewer), and
// keeps each thread's exclusive prefix in cum[t] (lane t covers ordered bins
// kBins - 1 - 2t and kBins - 2 - 2t), from which count_above() later reads
// the count above any bin without another scan.
__device__ __forceinline__ void two_thresholds_raw(const uint32_t* hist, uint32_t need1, uint32_t need2,
                                                   uint32_t* scratch, uint32_t* cum, uint32_t* b1, uint32_t* b2) {
  constexpr int PB = kBins / kBlock;
  const int t = threadIdx.x;
  uint32_t h[PB], s = 0;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const uint32_t b = (uint32_t)(kBins - 1 - (t * PB + j));
    h[j] = (b >= kFirstBin && b <= kLastBin) ? hist[raw_of_bin(b)] : 0u;
    s += h[j];
  }
  uint32_t c = block_exclusive_add(s, scratch);
  cum[t] = c;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const uint32_t b = (uint32_t)(kBins - 1 - (t * PB + j));
    if (c < need1 && need1 <= c + h[j]) *b1 = b;
    if (c < need2 && need2 <= c + h[j]) *b2 = b;
    c += h[j];
  }
  __syncthreads();
}

// Scores of the chunk in bins above ordered bin b, from two_thresholds_raw's
// prefixes (uniform: every lane reads the same words).
__device__ __forceinline__ uint32_t count_above(const uint32_t* hist, const uint32_t* cum, uint32_t b) {
  constexpr int PB = kBins / kBlock;
  static_assert(PB == 2, "two bins per lane");
  const uint32_t from_top = (uint32_t)(kBins - 1) - b;
  const uint32_t tb = from_top / PB;
  uint32_t above = cum[tb];
  if (from_top % PB) {
    const uint32_t b0 = (uint32_t)(kBins - 1) - tb * PB;
    above += (b0 >= kFirstBin && b0 <= kLastBin) ? hist[raw_of_bin(b0)] : 0u;
  }
  return uni(above);
}

// Compressed composite key of a boundary candidate: the FP32 key offset from
// the smallest candidate key, then the position reversed so that lower
// positions rank higher. Distinct for distinct positions, so the top `need`
// keys are unique, and the position is recoverable from the low b2 bits.
struct Refine {
  uint32_t lo32;
  uint32_t b2;      // bits of the reversed position
  uint32_t idx_hi;  // largest candidate position
  uint32_t nb;      // total key bits
  uint32_t need;    // boundary elements still to select
  uint32_t cnt;     // boundary elements in total
  __device__ __forceinline__ uint64_t key(uint32_t k32, int32_t i) const {
    return ((uint64_t)(k32 - lo32) << b2) | (uint64_t)(idx_hi - (uint32_t)i);
  }
  __device__ __forceinline__ int32_t pos(uint64_t ck) const {
    return (int32_t)(idx_hi - (uint32_t)(ck & ((1ull << b2) - 1ull)));
  }
};

__device__ __forceinline__ uint32_t bit_width(uint32_t x) { return x ? 32u - (uint32_t)__clz(x) : 0u; }

// From the candidate range (kmax, ~kmin, imax, ~imin).
__device__ __forceinline__ Refine make_refine(const uint32_t* range, uint32_t need, uint32_t cnt) {
  Refine p;
  const uint32_t kmax = uni(range[0]), kmin = ~uni(range[1]), imax = uni(range[2]), imin = ~uni(range[3]);
  p.lo32 = kmin;
  p.idx_hi = imax;
  p.b2 = bit_width(imax - imin);
  p.nb = bit_width(kmax - kmin) + p.b2;
  p.need = need;
  p.cnt = cnt;
  return p;
}

// FP32-key digit of a threshold-bin candidate in a frame that depends on the
// bin alone, so every workgroup of a split row computes the same digit
// without another exchange. A score whose FP16 rounding lies in ordered bin
// b lies strictly between the FP16 values just below and just above the bin
// (rounding is monotone and both are exactly representable in FP32), so its
// key32 lies in [lo, hi] with lo, hi the keys of those two values (the key of
// -0 is the key of +0, hence not strictly). Beyond -inf or +inf (NaN codes)
// the frame runs to the end of the key range. The digit is the key offset
// from lo shifted right until the frame fits 13 bits, clamped: a monotone
// function of the key, so a digit above another means a larger score.
struct FineFrame {
  uint32_t lo;
  uint32_t shift;
  __device__ __forceinline__ uint32_t digit(uint32_t key) const {
    const uint32_t d = key >= lo ? (key - lo) >> shift : 0u;
    return min(d, (uint32_t)kFineBins - 1u);
  }
};
__device__ __forceinline__ bool key16_is_nan(uint32_t key16) {
  const uint32_t h = half_bits_of_key16(key16);
  return (h & 0x7C00u) == 0x7C00u && (h & 0x03FFu) != 0u;
}
__device__ __forceinline__ uint32_t key32_of_key16(uint32_t key16) {
  return key32_of((float)half_of_bits(half_bits_of_key16(key16)));
}
// b is a threshold bin, so kFirstBin <= b <= kLastBin: both neighbours are
// 16-bit codes.
__device__ __forceinline__ FineFrame fine_frame(uint32_t b) {
  const uint32_t below = b * 64u - 1u, above = b * 64u + 64u;
  FineFrame f;
  f.lo = key16_is_nan(below) ? 0u : key32_of_key16(below);
  const uint32_t hi = key16_is_nan(above) ? 0xFFFFFFFFu : key32_of_key16(above);
  const uint32_t w = bit_width(hi - f.lo);
  f.shift = w > (uint32_t)kFineBits ? w - (uint32_t)kFineBits : 0u;
  return f;
}
// The composite key of a threshold-bin candidate in its fine digit's frame:
// ((key32 - lo) << b2) | (len - 1 - position), with b2 = bitwidth(len - 1)
// and 13 + shift key bits (every candidate's key offset is below
// 2^(13 + shift)), so its top 13 bits are its fine digit. It depends on the
// threshold bin and the row length alone, so every workgroup of a split row
// derives the same one; their producers store candidates in this form.
__device__ __forceinline__ Refine fine_key_frame(FineFrame fr, uint32_t len) {
  Refine p;
  p.lo32 = fr.lo;
  p.idx_hi = len - 1u;
  p.b2 = bit_width(len - 1u);
  p.nb = (uint32_t)kFineBits + fr.shift + p.b2;
  p.need = 0;
  p.cnt = 0;
  return p;
}

// Split rows whose threshold bin holds more candidates than this count them
// by fine digit as they classify (below it the last workgroup's register pass
// is cheap), up to what that pass holds in registers.
constexpr uint32_t kFineMin = 4096;

// --- candidate sources for the exact refinement -----------------------------
// each(f) calls f(valid, composite key) for every element slot; the trip count
// is uniform across the workgroup so wave-level ballots stay convergent.

// Composite keys already in LDS.
struct KeyListSrc {
  static constexpr bool kStream = false;
  const uint64_t* p;
  uint32_t n;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (uint32_t i0 = 0; i0 < n; i0 += kBlock) {
      const uint32_t i = i0 + threadIdx.x;
      const bool valid = i < n;
      f(valid, valid ? p[i] : 0ull);
    }
  }
};

// (key32 << 32 | position) pairs that other workgroups left in global memory,
// read with device-coherent loads.
struct PairListSrc {
  static constexpr bool kStream = false;
  const uint64_t* p;
  uint32_t n;
  Refine r;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (uint32_t i0 = 0; i0 < n; i0 += kBlock) {
      const uint32_t i = i0 + threadIdx.x;
      const bool valid = i < n;
      const uint64_t e = valid ? ld_agent(p + i) : 0ull;
      f(valid, r.key((uint32_t)(e >> 32), (int32_t)(uint32_t)e));
    }
  }
};

// Threshold-bin scores of [begin, end), re-read from the row. Each step
// loads kStreamVec dwordx4 per lane (all in flight together) before using
// any of them, so a pass over the row is a few long bursts rather than many
// short round trips.
constexpr int kStreamVec = 8;

// FIRST: the first emission pass takes emit_first_digit (the streamed kernel
// variants' owned rows; elsewhere it would only add registers).
template <bool VEC, bool FIRST = false>
struct StreamSrc {
  static constexpr bool kStream = FIRST;
  const float* rowp;
  int32_t begin, end;
  Cut cut;
  Refine r;
  // The exact selection's first emission pass over the row when its digit
  // lies above the position bits (key offset >> ks, masked; the frame holds
  // offsets below 2^kw): scores in the frame with a digit above d (or equal
  // to it when `finish`) are output, those equal to d kept in `list` when
  // `compact`. Each step's outputs and kept keys are reserved with one
  // cursor add per wave (a wave prefix of the lanes' counts) instead of one
  // per element, whose round trip each element would otherwise wait for.
  template <class O>
  __device__ __forceinline__ bool emit_first_digit(uint32_t ks, uint32_t kw, uint32_t mask, uint32_t d, bool finish,
                                                   bool compact, uint32_t* cur_out, uint32_t* cur_list,
                                                   uint64_t* list, const O& o) const {
    constexpr int V = kStreamVec / 2;   // 16 scores per lane and reservation
    constexpr int32_t kSpan = V * kBlock * 4;
    static_assert(V * 4 <= 32, "one bit per element of a step");
    bool bad = false;
    auto load = [&](float (&x)[V * 4], int32_t base) {
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int32_t e = base + (u * kBlock + (int)threadIdx.x) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) x[u * 4 + c] = 0.f;
        if constexpr (VEC) {
          if (e < end) {
            const float4 v = *reinterpret_cast<const float4*>(rowp + e);
            x[u * 4 + 0] = v.x;
            x[u * 4 + 1] = v.y;
            x[u * 4 + 2] = v.z;
            x[u * 4 + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (e + c < end) x[u * 4 + c] = rowp[e + c];
        }
      }
    };
    auto use = [&](const float (&x)[V * 4], int32_t base) {
      uint32_t tm = 0, km = 0;   // bit j: element j is output / kept
#pragma unroll
      for (int j = 0; j < V * 4; ++j) {
        const int32_t e = base + ((j >> 2) * kBlock + (int)threadIdx.x) * 4 + (j & 3);
        const _Float16 h = half_lo(to_half2(x[j], 0.f));
        const bool in_bin = e < end && h >= cut.vlo && !(h >= cut.vhi);
        const uint32_t off = key32_of(x[j]) - r.lo32;
        const bool m = in_bin && (uint64_t)off < (1ull << kw);
        const uint32_t dig = (off >> ks) & mask;
        tm |= (uint32_t)(m && (dig > d || (finish && dig == d))) << j;
        km |= (uint32_t)(compact && m && dig == d) << j;
      }
      const uint32_t nt = (uint32_t)__popc(tm), nk = (uint32_t)__popc(km);
      const uint32_t it = wave_inclusive_add(nt), ik = wave_inclusive_add(nk);
      const uint32_t tt = read_lane(it, kWave - 1), tk = read_lane(ik, kWave - 1);
      if ((tt | tk) == 0) return;   // (uniform)
      uint32_t bt = 0, bk = 0;
      if (lane() == 0) {
        if (tt) bt = atomicAdd(cur_out, tt);
        if (tk) bk = atomicAdd(cur_list, tk);
      }
      uint32_t ot = read_lane(bt, 0) + it - nt, ok = read_lane(bk, 0) + ik - nk;
#pragma unroll
      for (int j = 0; j < V * 4; ++j) {
        const int32_t e = base + ((j >> 2) * kBlock + (int)threadIdx.x) * 4 + (j & 3);
        if ((tm >> j) & 1u) bad |= !o.write(ot++, e);
        if ((km >> j) & 1u) list[ok++] = r.key(key32_of(x[j]), e);
      }
    };
    // The next step's loads are in flight while a step is used (two register
    // sets, the loop unrolled twice so that neither is copied).
    float xa[V * 4], xb[V * 4];
    int32_t base = begin;
    load(xa, base);
    for (;;) {
      if (base >= end) break;
      load(xb, base + kSpan);
      use(xa, base);
      base += kSpan;
      if (base >= end) break;
      load(xa, base + kSpan);
      use(xb, base);
      base += kSpan;
    }
    return bad;
  }
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (int32_t base = begin; base < end; base += kStreamVec * kBlock * 4) {
      float x[kStreamVec * 4];
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u) {
        const int32_t e = base + (u * kBlock + (int)threadIdx.x) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) x[u * 4 + c] = 0.f;
        if constexpr (VEC) {
          if (e < end) {
            const float4 v = *reinterpret_cast<const float4*>(rowp + e);
            x[u * 4 + 0] = v.x;
            x[u * 4 + 1] = v.y;
            x[u * 4 + 2] = v.z;
            x[u * 4 + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (e + c < end) x[u * 4 + c] = rowp[e + c];
        }
      }
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int32_t e = base + (u * kBlock + (int)threadIdx.x) * 4 + c;
          const _Float16 h = half_lo(to_half2(x[u * 4 + c], 0.f));
          const bool in_bin = e < end && h >= cut.vlo && !(h >= cut.vhi);
          f(in_bin, in_bin ? r.key(key32_of(x[u * 4 + c]), e) : 0ull);
        }
    }
  }
};

// Exact selection of the `need` best boundary candidates (FP32 value
// descending, position ascending): MSB-first radix over the composite key.
// Each pass histograms one digit of the candidates that match the prefix
// fixed so far, finds the digit holding the need-th, emits the candidates
// with a larger digit and keeps the equal ones; survivors are compacted into
// free LDS list space as soon as they fit. The first pass takes a 13-bit
// digit when 34 KB of the list are free for its (padded) histogram.
// Outputs are staged from sh.cur_out onwards. SRC_IN_LDS: the source is the
// composite-key list sh.list[0, n0). The search may resume after `pbits0`
// key bits already fixed to `prefix0`, with `need0` still to select.
// `counted`: the first pass's 13-bit histogram (padded, at the start of the
// list region) was already filled while the source was classified, so the
// first pass only emits and compacts (streamed sources, pbits0 == 0).
template <bool SRC_IN_LDS, class Src>
__device__ __forceinline__ void refine(const Src& src, const Refine& p, Smem& sh, const RowOut& o,
                                       uint64_t prefix0, uint32_t pbits0, uint32_t need0, uint32_t n0,
                                       bool counted = false) {
  const int t = threadIdx.x;
  bool bad = false;
  if (need0 == n0) {
    src.each([&](bool valid, uint64_t ck) {
      bad |= !emit_wave(valid && (ck >> (p.nb - pbits0)) == prefix0, p.pos(ck), &sh.cur_out, o);
    });
    report_bad(bad, o.status);
    __syncthreads();
    return;
  }
  uint64_t prefix = prefix0;
  uint32_t pbits = pbits0, need = need0;
  bool in_list = SRC_IN_LDS;
  uint32_t list_off = 0, list_n = SRC_IN_LDS ? n0 : 0u;   // current list: sh.list[list_off, +list_n)
  for (;;) {
    uint32_t* hist = sh.rhist;
    bool wide = false;
    if (pbits == 0) {
      if (!in_list) {
        hist = reinterpret_cast<uint32_t*>(sh.list);
        wide = true;
      } else if (list_off + list_n + kWideSlots <= (uint32_t)kListCap) {
        hist = reinterpret_cast<uint32_t*>(sh.list + list_off + list_n);
        wide = true;
      }
    }
    const uint32_t width = min(wide ? (uint32_t)kFirstRadixBits : (uint32_t)kRadixBits, p.nb - pbits);
    const uint32_t shift = p.nb - pbits - width;
    const uint32_t top = shift + width;   // <= 63
    const uint32_t mask = (1u << width) - 1u;
    const uint32_t words = wide ? (mask + 1) + ((mask + 1) >> kWidePad) : mask + 1;
    if (!counted) {
      for (int i = t; i < (int)words; i += kBlock) hist[i] = 0;
      __syncthreads();
      // Digits mix key and position bits, so hot bins are rare: plain atomics.
      auto hist_fn = [&](bool valid, uint64_t ck) {
        if (valid && (ck >> top) == prefix) {
          const uint32_t d = (uint32_t)(ck >> shift) & mask;
          atomicAdd(&hist[wide ? d + (d >> kWidePad) : d], 1u);
        }
      };
      if (in_list) KeyListSrc{sh.list + list_off, list_n}.each(hist_fn);
      else src.each(hist_fn);
    }
    counted = false;
    __syncthreads();
    if (t == 0) sh.res[0] = kNotFound;
    if (wide) find_threshold<kFirstRadixBins / kBlock, kWidePad>(hist, (int)(mask + 1), need, sh.scratch, sh.res);
    else find_threshold<kRadixBins / kBlock>(hist, (int)(mask + 1), need, sh.scratch, sh.res);
    const uint32_t d = uni(sh.res[0]), above = uni(sh.res[1]), cnt = uni(sh.res[2]);
    if (d == kNotFound) {
      if (t == 0) atomicOr(o.status, TOPK_DEVICE_INTERNAL);
      break;
    }
    const bool finish = cnt == need - above;
    // compaction target: the whole list when the source lies outside LDS,
    // else the free part before or after the current list
    uint32_t target = 0;
    bool compact = false;
    if (!finish) {
      if (!in_list) {
        compact = cnt <= (uint32_t)kListCap;
      } else if (list_off == 0) {
        target = list_n;
        compact = list_n + cnt <= (uint32_t)kListCap;
      } else {
        compact = cnt <= list_off;
      }
    }
    if (t == 0) sh.cur_list = target;
    __syncthreads();
    auto emit_fn = [&](bool valid, uint64_t ck) {
      const bool m = valid && (ck >> top) == prefix;
      const uint32_t dig = (uint32_t)(ck >> shift) & mask;
      bad |= !emit_wave(m && (dig > d || (finish && dig == d)), p.pos(ck), &sh.cur_out, o);
      if (compact) push_wave(m && dig == d, ck, &sh.cur_list, sh.list);
    };
    bool emitted = false;
    if constexpr (Src::kStream) {
      // The first pass over a streamed row, its digit above the position
      // bits (prefix empty, so only the frame test remains): per-step
      // reservations (StreamSrc::emit_first_digit).
      if (!in_list && pbits == 0 && shift >= p.b2) {
        bad |= src.emit_first_digit(shift - p.b2, p.nb - p.b2, mask, d, finish, compact, &sh.cur_out, &sh.cur_list,
                                    sh.list, o);
        emitted = true;
      }
    }
    if (!emitted) {
      if (in_list) KeyListSrc{sh.list + list_off, list_n}.each(emit_fn);
      else src.each(emit_fn);
    }
    __syncthreads();
    if (finish) break;
    need -= above;
    prefix = (prefix << width) | d;
    pbits += width;
    if (compact) {
      in_list = true;
      list_off = target;
      list_n = cnt;
    }
  }
  report_bad(bad, o.status);
}

template <bool SRC_IN_LDS, class Src>
__device__ __forceinline__ void refine(const Src& src, const Refine& p, Smem& sh, const RowOut& o) {
  refine<SRC_IN_LDS>(src, p, sh, o, 0ull, 0u, p.need, p.cnt);
}

// First refinement pass over n <= J * kBlock boundary candidates held in
// registers as 32-bit key offsets kd (FP32 key minus the smallest candidate
// key) and positions (lane t holds entries j * kBlock + t). The digit is 13
// bits for large sets, 11 for small ones; it comes from kd alone when the
// key range is at least that wide (the composite key's top bits are then key
// bits), else from the composite key. Its histogram, padded one word per
// lane-group so the threshold scan is bank-conflict free, lives in the (free)
// LDS list region; emission and compaction offsets come from one block scan
// of per-lane counts. Survivors continue in LDS as composite keys.
// CLEARED: the caller has already zeroed kWideWords words of the list (the
// largest histogram this pass uses).
template <int J, bool CLEARED = false>
__device__ __forceinline__ void resolve_regs(const uint32_t (&kd)[J], const uint32_t (&ps)[J], uint32_t n,
                                             const Refine& p, Smem& sh, const RowOut& o) {
  static_assert(J * kBlock + 2 * kBlock <= kListCap, "per-lane sink slots lie past the candidates");
  static_assert((kWideWords + kBlock) / 2 <= kListCap - 2 * kBlock, "histogram sinks precede the write sinks");
  const int t = threadIdx.x;
  const bool wide = n > 4096u;
  const uint32_t width = min(wide ? (uint32_t)kFirstRadixBits : (uint32_t)kRadixBits, p.nb);
  const uint32_t shift = p.nb - width;
  const uint32_t mask = (1u << width) - 1u;
  const uint32_t pad = wide ? 4u : 2u;   // log2 of the bins each lane scans
  // lane t holds nv valid entries: j * kBlock + t < n  <=>  j < nv
  const int nv = (int)((n + kBlock - 1 - (uint32_t)t) / kBlock);
  // Top `width` bits of the composite key (one formula whether or not they
  // reach into the position bits).
  // In 32-bit arithmetic: when the digit lies inside the key bits (shift >=
  // b2) it is kd >> (shift - b2); otherwise kd's bits shifted up by b2 - shift
  // join the top bits of the reversed position.
  const bool key_only = shift >= p.b2;
  const uint32_t sl = key_only ? 0u : p.b2 - shift;
  const uint32_t sr = key_only ? shift - p.b2 : 0u;
  const uint32_t rs = key_only ? 0u : shift;
  const uint32_t rm = key_only ? 0u : 0xFFFFFFFFu;
  // (Recomputed in each loop rather than held: an empty asm hides the value
  // from common-subexpression elimination, which would keep J digits live.)
  auto digit = [&](int j) -> uint32_t {
    uint32_t x = kd[j];
    asm volatile("" : "+v"(x));
    return (((x << sl) >> sr) | (((p.idx_hi - ps[j]) >> rs) & rm)) & mask;
  };
  uint32_t* hist = reinterpret_cast<uint32_t*>(sh.list);
  const uint32_t words = (mask + 1) + ((mask + 1) >> pad);
  if constexpr (!CLEARED) {
    for (int i = t; i < (int)words; i += kBlock) hist[i] = 0;
    __syncthreads();
  }
  // Invalid slots add into this lane's own sink word past the histogram (one
  // shared sink would serialise whole waves on a single address).
  const uint32_t sink = words + (uint32_t)t;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t d = digit(j);
    atomicAdd(&hist[j < nv ? d + (d >> pad) : sink], 1u);
  }
  __syncthreads();
  if (t == 0) sh.res[0] = kNotFound;
  if (wide) find_threshold<kFirstRadixBins / kBlock, 4>(hist, (int)(mask + 1), p.need, sh.scratch, sh.res);
  else find_threshold<kRadixBins / kBlock, 2>(hist, (int)(mask + 1), p.need, sh.scratch, sh.res);
  const uint32_t d = uni(sh.res[0]), above = uni(sh.res[1]), cnt = uni(sh.res[2]);
  if (d == kNotFound) {
    if (t == 0) atomicOr(o.status, TOPK_DEVICE_INTERNAL);
    return;
  }
  const bool finish = cnt == p.need - above;
  const uint32_t dlo = finish ? d : d + 1;   // emitted: digit >= dlo; kept (unless finish): digit == d
  const uint32_t dkeep = finish ? 0xFFFFFFFFu : d;
  uint32_t na = 0, nk = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t dj = digit(j);
    na += (j < nv && dj >= dlo) ? 1u : 0u;
    nk += (j < nv && dj == dkeep) ? 1u : 0u;
  }
  const uint32_t base = uni(sh.cur_out);
  uint32_t tot;
  const uint32_t off = block_exclusive_add((nk << 16) | na, sh.scratch, &tot);   // counts < 2^16
  const uint32_t total_out = tot & 0xFFFFu, total_keep = tot >> 16;
  // The counts bound every write, so one uniform check replaces per-element
  // bounds checks; unselected slots write to this lane's own sink entries past
  // the candidates (no branches, no bank conflicts among the sinks).
  const bool ok = base + total_out <= o.k && total_keep <= (uint32_t)(kListCap - 2 * kBlock);
  if (ok) {
    uint32_t* stage_sink = reinterpret_cast<uint32_t*>(sh.list + (kListCap - 2 * kBlock)) + t;
    uint64_t* list_sink = sh.list + (kListCap - kBlock) + t;
    uint32_t ao = base + (off & 0xFFFFu), ko = off >> 16;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t dj = digit(j);
      const bool em = j < nv && dj >= dlo;
      const bool kp = j < nv && dj == dkeep;
      *(em ? sh.outpos + ao : stage_sink) = ps[j];   // o.stage is sh.outpos
      *(kp ? sh.list + ko : list_sink) = p.key(kd[j] + p.lo32, (int32_t)ps[j]);
      ao += em ? 1u : 0u;
      ko += kp ? 1u : 0u;
    }
  }
  report_bad(!ok, o.status);
  __syncthreads();
  if (t == 0) sh.cur_out = base + total_out;
  __syncthreads();
  if (finish || !ok) return;
  refine<true>(KeyListSrc{sh.list, cnt}, p, sh, o, (uint64_t)d, width, p.need - above, cnt);
}

// Register slots per lane for n register-resident candidates.
constexpr int kRegSmall = 2, kRegMid = 8;
static_assert(kRegMid < kResolveRegs, "slot classes grow");

// Rewrite the LDS pair list sh.list[0, n) as composite keys, in place.
__device__ __forceinline__ void pairs_to_keys(Smem& sh, uint32_t n, const Refine& p) {
  for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
    const uint64_t e = sh.list[i];
    sh.list[i] = p.key((uint32_t)(e >> 32), (int32_t)(uint32_t)e);
  }
  __syncthreads();
}

// The pair list src[0, n) in LDS (default sh.list; n <= J * kBlock) into
// registers, then the register-resident first pass.
template <int J>
__device__ __forceinline__ void resolve_lds_pairs(uint32_t n, const Refine& p, Smem& sh, const RowOut& o,
                                                  const uint64_t* src = nullptr) {
  if (!src) src = sh.list;
  uint32_t kd[J], ps[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t i = (uint32_t)j * kBlock + threadIdx.x;
    const uint64_t v = i < n ? src[i] : 0ull;
    kd[j] = (uint32_t)(v >> 32) - p.lo32;
    ps[j] = (uint32_t)v;
  }
  __syncthreads();
  resolve_regs<J>(kd, ps, n, p, sh, o);
}

// A row the workgroup owns alone: register path when the row fits one tile,
// streaming path otherwise. Selected positions are staged in LDS and the
// row's k outputs flushed once at the end.
// Threshold-bin candidates that all hold one FP32 key (so one score): the
// `need` of them at the lowest positions are the selected ones. One pass in
// position order, kFirstGroups vector groups (kFirstGroups * 2,048
// positions) per step: a step whose candidates all fit the remaining need is
// emitted whole; in the step where the count is reached its vector groups
// are ranked one at a time (group q holds positions [2048 q, 2048 (q + 1))
// of the step, lane-major). The pass stops there, so the rest of the row is
// not read. Output slots come from block scans of the lanes' counts.
constexpr int kFirstGroups = 4;
template <bool VEC>
__device__ __forceinline__ void first_need(const float* rowp, int32_t len, Cut cut, uint32_t need, Smem& sh,
                                           const RowOut& o) {
  constexpr int32_t kStepLen = kFirstGroups * kBlock * 4;
  bool bad = false;
#pragma unroll 1
  for (int32_t base = 0; base < len && need > 0; base += kStepLen) {
    float4 x[kFirstGroups];
#pragma unroll
    for (int u = 0; u < kFirstGroups; ++u) {
      const int32_t e = tile_pos(base, u, 0);
      x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (VEC) {
        if (e < len) x[u] = *reinterpret_cast<const float4*>(rowp + e);
      } else {
        if (e < len) x[u].x = rowp[e];
        if (e + 1 < len) x[u].y = rowp[e + 1];
        if (e + 2 < len) x[u].z = rowp[e + 2];
        if (e + 3 < len) x[u].w = rowp[e + 3];
      }
    }
    // bit 4 u + j: the lane's position tile_pos(base, u, j) is a candidate
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < kFirstGroups; ++u) {
      const int32_t e = tile_pos(base, u, 0);
      const float v[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const _Float16 h = half_lo(to_half2(v[j], v[j]));
        m |= (e + j < len && h >= cut.vlo && !(h >= cut.vhi)) ? 1u << (4 * u + j) : 0u;
      }
    }
    const uint32_t cur = uni(sh.cur_out);
    uint32_t tot;
    uint32_t pos = cur + block_exclusive_add((uint32_t)__popc(m), sh.scratch, &tot);
    tot = uni(tot);
    if (tot <= need) {
      for (uint32_t mm = m; mm != 0; mm &= mm - 1) {
        const int b = __builtin_ctz(mm);
        bad |= !o.write(pos++, tile_pos(base, b >> 2, b & 3));
      }
      if (threadIdx.x == 0) sh.cur_out = cur + tot;
      need -= tot;
      __syncthreads();
      continue;
    }
    uint32_t done = 0;
#pragma unroll 1
    for (int u = 0; u < kFirstGroups && done < need; ++u) {
      const uint32_t mu = (m >> (4 * u)) & 0xFu;
      uint32_t tu;
      uint32_t r = done + block_exclusive_add((uint32_t)__popc(mu), sh.scratch, &tu);
      for (uint32_t mm = mu; mm != 0; mm &= mm - 1) {
        const int j = __builtin_ctz(mm);
        if (r < need) bad |= !o.write(cur + r, tile_pos(base, u, j));
        ++r;
      }
      done += uni(tu);
    }
    if (threadIdx.x == 0) sh.cur_out = cur + need;
    need = 0;
  }
  report_bad(bad, o.status);
  __syncthreads();
}

template <bool VEC, bool STREAM>
__device__ __forceinline__ void owned_row(const SelectArgs& a, int32_t len, const float* rowp, const RowOut& o,
                                          bool resident, uint32_t (&hk)[kHk], Smem& sh) {
  if (threadIdx.x == 0) sh.res[0] = kNotFound;
  find_threshold_raw(sh.lhist, (uint32_t)a.k, sh.scratch, sh.res);
  const uint32_t bstar = uni(sh.res[0]), n_above = uni(sh.res[1]), cnt = uni(sh.res[2]);
  if (bstar == kNotFound) {  // fewer valid scores than k: NaN inputs
    if (threadIdx.x == 0) atomicOr(a.status, TOPK_DEVICE_INTERNAL);
    return;
  }
  const Cut cut = cut_of_bin(bstar);
  const bool use_list = cnt <= (uint32_t)kListCap;
  // Too many candidates for the list: they are counted by the 13-bit digit of
  // their composite key in the threshold bin's fine frame as they are
  // classified, into the padded histogram the exact selection's first pass
  // uses (at the start of the free list region), so that pass needs no count
  // of its own over the row.
  const Refine pf = fine_key_frame(fine_frame(bstar), (uint32_t)len);
  // (the digit, the composite key's top 13 bits, is the key offset's top
  // bits: the position bits lie below them)
  const uint32_t fshift = pf.nb - (uint32_t)kFineBits - pf.b2;
  uint32_t* whist = reinterpret_cast<uint32_t*>(sh.list);
  if (!use_list)
    for (int i = threadIdx.x; i < kWideWords; i += kBlock) whist[i] = 0;
  if (threadIdx.x == 0) {
    sh.cur_out = 0;
    sh.cur_list = 0;
    sh.range[0] = sh.range[1] = sh.range[2] = sh.range[3] = 0;
  }
  __syncthreads();
  Range rg;
  bool bad = false;
  auto on_above = [&](int32_t e, int32_t) { bad |= !o.write(atomicAdd(&sh.cur_out, 1u), e); };
  auto on_cand = [&](uint32_t kk, int32_t e) {
    if (use_list) {
      const uint32_t c = atomicAdd(&sh.cur_list, 1u);
      const bool ok = c < (uint32_t)kListCap;
      if (ok) sh.list[c] = ((uint64_t)kk << 32) | (uint32_t)e;
      bad |= !ok;
    } else {
      // (one add per wave when its lanes share the digit: single-key rows)
      const uint32_t d = (kk - pf.lo32) >> fshift;
      hist_add(whist, true, d + (d >> kWidePad));
    }
  };
  if (resident) {
    extract(interest_mask(hk, cut.vlo), 0, rowp, cut.vhi, rg, on_above, on_cand);
  } else {
    // Streamed row. When many of its scores lie at or above the threshold
    // bin (dense boundary bins), each tile is read again whole and
    // classified from the FP32 registers; otherwise the tile is binned again
    // and only its few such positions are re-read.
    const bool dense = (uint64_t)(n_above + cnt) * 8u > (uint64_t)len;
    for (int32_t base = 0; base < len; base += kTile) {
      if (VEC && dense && !use_list) {
        // Every score is classified without branches: the above-threshold
        // ones are written through one wave-aggregated cursor add, the
        // candidates counted by digit (one add per wave when the lanes share
        // the digit), and only the key range is kept (the exact passes use
        // the fine frame, not the candidates' position range). (Rows read
        // with scalar loads keep the branching form, which needs no scratch
        // there.)
        float4 x[kEpt / 4];
        load_raw<VEC>(rowp, base, len, x);
#pragma unroll
        for (int q = 0; q < kEpt / 4; ++q) {
          const float xs[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
          bool above[4], cand[4];
          uint32_t dp[4];   // padded digit slots
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int32_t e = tile_pos(base, q, c);
            const _Float16 h = half_lo(to_half2(xs[c], xs[c]));
            const bool in = e < len;
            above[c] = in && h >= cut.vhi;
            cand[c] = in && !(h >= cut.vhi) && h >= cut.vlo;
            const uint32_t kk = key32_of(xs[c]);
            rg.kmax = max(rg.kmax, cand[c] ? kk : 0u);
            rg.kmin_inv = max(rg.kmin_inv, cand[c] ? ~kk : 0u);
            const uint32_t d = (kk - pf.lo32) >> fshift;
            dp[c] = d + (d >> kWidePad);
          }
          // (per vector: the outputs only where a lane has one, and one add
          // per wave when every lane's four scores share a digit)
          if (__ballot(above[0] || above[1] || above[2] || above[3])) {
#pragma unroll
            for (int c = 0; c < 4; ++c) bad |= !emit_wave(above[c], tile_pos(base, q, c), &sh.cur_out, o);
          }
          const uint32_t f = (uint32_t)__builtin_amdgcn_readfirstlane((int)dp[0]);
          const bool same = cand[0] && cand[1] && cand[2] && cand[3] && dp[0] == f && dp[1] == f && dp[2] == f &&
                            dp[3] == f;
          if (__ballot(same) == ~0ull) {
            if (lane() == 0) atomicAdd(&whist[f], 256u);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (cand[c]) atomicAdd(&whist[dp[c]], 1u);
          }
        }
      } else if (dense) {
        float4 x[kEpt / 4];
        load_raw<VEC>(rowp, base, len, x);
#pragma unroll
        for (int q = 0; q < kEpt / 4; ++q) {
          const int32_t e = tile_pos(base, q, 0);
          if (e < len) classify(x[q].x, e, 0, cut, rg, on_above, on_cand);
          if (e + 1 < len) classify(x[q].y, e + 1, 0, cut, rg, on_above, on_cand);
          if (e + 2 < len) classify(x[q].z, e + 2, 0, cut, rg, on_above, on_cand);
          if (e + 3 < len) classify(x[q].w, e + 3, 0, cut, rg, on_above, on_cand);
        }
      } else {
        load_pack<VEC>(rowp, base, len, hk);
        extract(interest_mask(hk, cut.vlo), base, rowp, cut.vhi, rg, on_above, on_cand);
      }
    }
  }
  merge_range(rg, sh);
  report_bad(bad, a.status);
  __syncthreads();
  const uint32_t need = (uint32_t)a.k - n_above;
  const Refine p = make_refine(sh.range, need, cnt);
  if (STREAM && !resident && !use_list && uni(sh.range[0]) == ~uni(sh.range[1])) {
    // Every candidate holds the same FP32 key: the lowest positions win.
    // (Streamed rows only: in a row of one tile the fine-digit passes below
    // cost a tile read each, and the extra pass would only add registers to
    // the kernels that serve such rows.)
    if constexpr (STREAM) first_need<VEC>(rowp, len, cut, need, sh, o);
  } else if (!use_list) {
    Refine q = pf;
    q.need = need;
    q.cnt = cnt;
    refine<false>(StreamSrc<VEC, STREAM>{rowp, 0, len, cut, q}, q, sh, o, 0ull, 0u, need, cnt, true);
  } else if (cnt <= (uint32_t)(kRegSmall * kBlock)) {
    resolve_lds_pairs<kRegSmall>(cnt, p, sh, o);
  } else if (cnt <= (uint32_t)(kRegMid * kBlock)) {
    resolve_lds_pairs<kRegMid>(cnt, p, sh, o);
  } else if (cnt <= (uint32_t)(kResolveRegs * kBlock)) {
    resolve_lds_pairs<kResolveRegs>(cnt, p, sh, o);
  } else {
    pairs_to_keys(sh, cnt, p);
    refine<true>(KeyListSrc{sh.list, cnt}, p, sh, o);
  }
  report_bad(!o.flush(0, (uint32_t)a.k), a.status);
}

// The last workgroup of a split row resolves its threshold bin from the
// candidates the row's workgroups left in global memory, then flushes the
// outputs [n_above, k). The candidate range and (when they fit the
// registers) the candidates are fetched in one round trip.
// Candidates [0, n) of a split row's global list (n <= J * kBlock) and the
// row's candidate range, fetched in one round trip; then the register pass.
template <int J>
__device__ __forceinline__ void resolve_global_regs(const GroupState* g, const uint64_t* slab, uint32_t need,
                                                    uint32_t n, Smem& sh, const RowOut& o) {
  const int t = threadIdx.x;
  uint64_t e[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t i = (uint32_t)j * kBlock + t;
    e[j] = i < n ? ld_agent(slab + i) : 0ull;
  }
  const uint32_t rng = t < 4 ? ld_agent(&g->range[t]) : 0u;
  // The first pass's histogram is cleared while the candidates arrive.
  static_assert(kWideWords % 4 == 0, "cleared in 16-byte stores");
  for (int i = t; i < kWideWords / 4; i += kBlock) reinterpret_cast<uint4*>(sh.list)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (t < 4) sh.range[t] = rng;
  __syncthreads();
  const Refine p = make_refine(sh.range, need, n);
  uint32_t kd[J], ps[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    kd[j] = (uint32_t)(e[j] >> 32) - p.lo32;
    ps[j] = (uint32_t)e[j];
  }
  resolve_regs<J, true>(kd, ps, n, p, sh, o);
}

// Whole workgroup: copy n 64-bit words that other workgroups wrote (agent
// scope) from src to LDS dst with direct-to-LDS loads (global_load_lds, 16
// bytes per lane, cache policy sc1 = device coherent), so the data in flight
// holds no registers. Each wave instruction moves 128 consecutive words; lanes
// past n re-read the last word (in bounds) into slots past n, so dst must have
// room for n rounded up to 128. The caller waits (vmcnt) and synchronises.
constexpr int kLdsCopyWords = kWave * 2;   // 64-bit words per wave instruction
__device__ __forceinline__ void copy_agent_to_lds(const uint64_t* src, uint32_t n, uint64_t* dst) {
  if (n == 0) return;
  const uint32_t w = uni(threadIdx.x >> 6);
  for (uint32_t base = w * kLdsCopyWords; base < n; base += kWaves * kLdsCopyWords) {
    const uint32_t i = min(base + 2u * lane(), (n - 1u) & ~1u);   // even, so the 16-byte load stays aligned
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + i),
                                     (__attribute__((address_space(3))) void*)(dst + base), 16, 0, 16);
  }
}

// A fine row's last workgroup copies up to kFineMaxCand candidates to the LDS
// list, then the digit counts above them.
constexpr uint32_t kFineMaxCand = kResolveRegs * kBlock;      // 12,288 candidates ...
constexpr uint32_t kFineHistEntry = kFineMaxCand;             // ... then the digit counts
static_assert(kFineHistEntry + kFineBins / 2 <= (uint32_t)kListCap, "candidates and digit counts share the LDS list");
static_assert(kFineMaxCand % kLdsCopyWords == 0, "the rounded-up copy stays below the digit counts");

// A workgroup's fine-digit counts in LDS go to the row's digit histogram, one
// atomic per nonzero digit; once this wave's atomics have landed (its own
// wait), the digit groups' sums go to the row's coarse counts. A reader that
// finds the coarse counts complete therefore also reads a complete digit
// histogram, and polls 128 words instead of 8,192. Wave w takes digits
// 512 j + 64 w + lane: one instruction adds a whole group of 64 consecutive
// digits, which the memory system merges per cache line (one digit per
// instruction, hot digits shared by every workgroup of the row serialise
// there instead); the group sums were counted in LDS with the digits
// (lfine[kFineBins + group]), and lane j of wave w adds group 8 j + w.
static_assert(kFineBins == 16 * kBlock && kFineGroups * 64 == kFineBins, "16 digit groups per wave");
__device__ __forceinline__ void merge_fine(const uint32_t* lfine, GroupState* g) {
  const int t = threadIdx.x;
  const uint32_t w = uni((uint32_t)t >> 6);
#pragma unroll 8
  for (int j = 0; j < kFineBins / kBlock; ++j) {
    const int d = j * kBlock + t;
    const uint32_t c = lfine[d];
    if (c) __hip_atomic_fetch_add(&g->fine[d], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const uint32_t sum = lane() < 16u ? lfine[kFineBins + lane() * kWaves + w] : 0u;
  drain_memory();
  if (sum)
    __hip_atomic_fetch_add(&g->fine_c[lane() * kWaves + w], sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// How a workgroup's fine-digit counts reach the row (fine_tail):
enum FineMerge {
  kFineMerged = 0,   // already merged (classified before the histogram wait)
  kFineInLds = 1,    // digit counts in LDS at kFineListOff
  kFineGlobal = 2,   // digits added to the row's histogram directly, group sums in LDS (lhist)
};

// Every workgroup of a split row whose threshold bin holds more than
// kFineMin candidates ("fine" rows), after classifying its chunk: its
// candidates sit in the LDS list as fine-frame composite keys (fine_key_frame)
// and its fine-digit counts in LDS (fine_lds) or already in the row's digit
// histogram. It adds its nonzero counts to the row's histogram (one atomic
// each; a few hundred per workgroup), then reads that histogram until the
// counts sum to the threshold bin's total: every
// contribution only adds, so a read that reaches the total has read every
// final count (the snapshot argument of the first wait). A scan from the top
// finds the digit d* holding the need-th largest candidate. Each workgroup
// then selects its own candidates above d* (all of d* when every candidate
// there is needed) and sends only those in d* to the row's list; the last
// workgroup resolves those few exactly and flushes the rest of the outputs.
template <bool VEC>
__device__ __forceinline__ void fine_tail(const SelectArgs& a, GroupState* g, uint64_t* slab, int32_t len,
                                          uint32_t G, uint32_t k, uint32_t n_above, uint32_t cnt,
                                          uint32_t local_above, int merge, Refine p, Smem& sh,
                                          const RowOut& o, bool bad, uint32_t* staged, uint32_t* staged_pg,
                                          uint32_t surv_cap) {
  const int t = threadIdx.x;
  const uint32_t w = uni((uint32_t)t >> 6);
  const uint32_t need = k - n_above;
  const uint32_t* lfine = reinterpret_cast<const uint32_t*>(sh.list + kFineListOff);
  if (merge == kFineGlobal) drain_memory();   // (this wave's digit atomics land before the group sums go)
  __syncthreads();   // classification complete (staged list, digit counts, above-threshold outputs)
  if (merge == kFineInLds) merge_fine(lfine, g);
  if (merge == kFineGlobal && t < kFineGroups && sh.lhist[t])
    __hip_atomic_fetch_add(&g->fine_c[t], sh.lhist[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // Poll the coarse counts (lane t < 128 holds group 127 - t: thread order
  // runs from the top group down) until they add up to the threshold bin's
  // total: every contribution only adds, so a read that reaches the total
  // has read every final count (the snapshot argument of the first wait),
  // and every digit behind them has landed.
  bool ok = false;
  uint32_t gc = 0, gcum = 0;
  for (uint32_t spins = 0; spins < a.spin_limit; ++spins) {
    gc = t < kFineGroups ? ld_agent(&g->fine_c[kFineGroups - 1 - t]) : 0u;
    uint32_t tot;
    gcum = block_exclusive_add(gc, sh.scratch, &tot);   // candidates in the groups above this lane's
    if (uni(tot) == cnt) {
      ok = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ok) {
    if (t == 0) atomicOr(a.status, TOPK_DEVICE_SPIN_TIMEOUT);
    return;
  }
  if (t == 0) sh.res[0] = sh.res[2] = kNotFound;
  __syncthreads();
  if (t < kFineGroups && gcum < need && need <= gcum + gc) {
    sh.res[0] = (uint32_t)(kFineGroups - 1 - t);
    sh.res[1] = gcum;
  }
  __syncthreads();
  // The group holding the need-th candidate: one wave reads its 64 digits,
  // top first, and finds d* with a wave prefix sum.
  const uint32_t grp = uni(sh.res[0]);
  if (grp != kNotFound && t < kWave) {
    const uint32_t d = grp * 64u + 63u - (uint32_t)t;
    const uint32_t h = ld_agent(&g->fine[d]);
    const uint32_t c = uni(sh.res[1]) + wave_inclusive_add(h) - h;
    if (c < need && need <= c + h) {
      sh.res[2] = d;
      sh.res[3] = c;
      sh.bcast[3] = h;
    }
  }
  __syncthreads();
  const uint32_t dstar = uni(sh.res[2]), above = uni(sh.res[3]), cnt_d = uni(sh.bcast[3]);
  const bool found = dstar != kNotFound;
  const bool all_of_d = found && cnt_d == need - above;
  const uint32_t dsel = all_of_d ? dstar : dstar + 1u;
  const uint32_t dshift = p.nb - (uint32_t)kFineBits;
  // This workgroup's candidates, each wave a contiguous share: counted first
  // (ballots), then one atomic per row cursor reserves the workgroup's
  // outputs and survivors, and the second pass writes them.
  const uint32_t n_c = found ? min(uni(sh.cur_list), (uint32_t)kStageCap) : 0u;
  const uint32_t per = ((n_c + kWaves - 1) / kWaves + kWave - 1) / kWave * kWave;
  const uint32_t lo = min(w * per, n_c), hi = min(lo + per, n_c);
  uint32_t nsel = 0, nkeep = 0;   // (uniform)
  for (uint32_t i0 = lo; i0 < hi; i0 += kWave) {
    const uint32_t i = i0 + lane();
    const uint64_t v = i < hi ? sh.list[i] : 0ull;
    const uint32_t d = (uint32_t)(v >> dshift);
    nsel += (uint32_t)__popcll(__ballot(i < hi && d >= dsel));
    nkeep += (uint32_t)__popcll(__ballot(i < hi && !all_of_d && d == dstar));
  }
  if (lane() == 0) {
    reinterpret_cast<uint32_t*>(sh.pl_red)[w] = nsel;
    reinterpret_cast<uint32_t*>(sh.pl_red)[kWaves + w] = nkeep;
  }
  __syncthreads();
  uint32_t bsel = 0, bkeep = 0, tsel = 0, tkeep = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t cs = reinterpret_cast<const uint32_t*>(sh.pl_red)[i];
    const uint32_t ck = reinterpret_cast<const uint32_t*>(sh.pl_red)[kWaves + i];
    bsel += (uint32_t)i < w ? cs : 0u;
    bkeep += (uint32_t)i < w ? ck : 0u;
    tsel += cs;
    tkeep += ck;
  }
  const uint32_t n_above_loc = min(uni(sh.cur_out), (uint32_t)kMaxK);   // staged above-threshold outputs
  if (t == 0) {
    // (the opaque zero keeps the plain fetch-add form: see the early atomics)
    const uint32_t z = opaque_zero();
    uint32_t bo = 0, bc = 0;
    if (local_above + tsel) bo = __hip_atomic_fetch_add(&g->emit + z, local_above + tsel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tkeep) bc = __hip_atomic_fetch_add(&g->cand + z, tkeep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.bcast[0] = bo;
    sh.bcast[1] = bc;
  }
  // Selected candidates join the staged outputs (their table entries are
  // read below); survivors are staged past the candidates, or, when they do
  // not fit there, stored to the row's list once the reservation returns.
  const uint32_t surv_off = (n_c + 1u) & ~1u;
  const bool room = n_above_loc + tsel <= (uint32_t)kMaxK;
  const bool stage_surv = surv_off + tkeep <= surv_cap;
  if (!stage_surv) __syncthreads();
  const uint32_t bc_direct = stage_surv ? 0u : uni(sh.bcast[1]);
  if (room) {
    uint32_t ao = n_above_loc + bsel, ko = bkeep;
    for (uint32_t i0 = lo; i0 < hi; i0 += kWave) {
      const uint32_t i = i0 + lane();
      const uint64_t v = i < hi ? sh.list[i] : 0ull;
      const uint32_t d = (uint32_t)(v >> dshift);
      const bool sel = i < hi && d >= dsel, kp = i < hi && !all_of_d && d == dstar;
      const uint64_t ms = __ballot(sel), mk = __ballot(kp);
      if (sel) staged[ao + mbcnt(ms)] = (uint32_t)p.pos(v);
      if (kp) {
        const uint32_t j = ko + mbcnt(mk);
        if (stage_surv) {
          sh.list[surv_off + j] = v;
        } else {
          const bool fits = (int64_t)(bc_direct + j) < a.cand_cap;
          if (fits) st_agent(slab + bc_direct + j, v);
          bad |= !fits;
        }
      }
      ao += (uint32_t)__popcll(ms);
      ko += (uint32_t)__popcll(mk);
    }
  }
  bad |= !room || (found && tkeep > cnt_d);
  __syncthreads();
  // Stores: the outputs (table entries of the selected candidates read now,
  // in flight with the reservation's round trip) and the survivors.
  // (survivors first: only they must have landed before the arrival count;
  // waves 1 to 7 store the outputs during the round trip of `done`)
  const uint32_t n_out = room ? n_above_loc + tsel : n_above_loc;
  const uint32_t bo = uni(sh.bcast[0]), bc = uni(sh.bcast[1]);
  if (room && stage_surv)
    for (uint32_t i = t; i < tkeep; i += kBlock) {
      const bool fits = (int64_t)(bc + i) < a.cand_cap;
      if (fits) st_agent(slab + bc + i, sh.list[surv_off + i]);
      bad |= !fits;
    }
  drain_memory();
  __syncthreads();
  if (t == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&g->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = prev == G - 1u;
  } else if (t >= kWave) {
    for (uint32_t i = t - kWave; i < n_out; i += kBlock - kWave) {
      const int32_t e = (int32_t)staged[i];
      const int32_t pg = i < n_above_loc ? (int32_t)staged_pg[i] : ((uint32_t)e < (uint32_t)len ? o.page(e) : 0);
      bad |= !o.store_page(bo + i, e, pg);
    }
  }
  report_bad(bad, a.status);
  __syncthreads();
  if (!uni(sh.flag)) return;
  // The last workgroup: d*'s survivors (cnt_d, all in the list now) resolved
  // exactly below the 13 bits fixed to d*, then the row's state left zeroed.
  if (found && !all_of_d) {
    if (t == 0) sh.cur_out = n_above + above;
    copy_agent_to_lds(slab, cnt_d, sh.list);
    drain_memory();
    __syncthreads();
    p.need = need - above;
    p.cnt = cnt_d;
    refine<true>(KeyListSrc{sh.list, cnt_d}, p, sh, o, (uint64_t)dstar, (uint32_t)kFineBits, need - above, cnt_d);
    report_bad(!o.flush(n_above + above, k), o.status);
  }
  if (!found && t == 0) atomicOr(a.status, TOPK_DEVICE_INTERNAL);
  uint64_t* fg = reinterpret_cast<uint64_t*>(g->fine);
  for (int i = t; i < kFineBins / 2; i += kBlock) st_agent(fg + i, (uint64_t)0);
  if (t < kFineGroups) st_agent(&g->fine_c[t], 0u);
  for (int r = t; r < kBins; r += kBlock) st_agent(&g->hist[r], 0u);
  if (t < 4) st_agent(&g->range[t], 0u);
  if (t == 0) {
    st_agent(&g->arrive, (uint64_t)0);
    st_agent(&g->vsq, (uint64_t)0);
    st_agent(&g->emit, 0u);
    st_agent(&g->cand, 0u);
    st_agent(&g->done, 0u);
  }
}

// The last workgroup of a split row resolves its threshold bin from the
// candidates the row's workgroups left in global memory, then flushes the
// outputs [n_above, k).
template <bool VEC>
__device__ __forceinline__ void resolve_split(const SelectArgs& a, GroupState* g, const uint64_t* slab,
                                              bool keep, int32_t len, const float* rowp,
                                              Cut cut, uint32_t need, uint32_t cnt, uint32_t n_above, Smem& sh,
                                              const RowOut& o) {
  const int t = threadIdx.x;
  if (t == 0) sh.cur_out = n_above;
  if (keep && cnt <= (uint32_t)(kRegSmall * kBlock)) {
    resolve_global_regs<kRegSmall>(g, slab, need, cnt, sh, o);
  } else if (keep && cnt <= (uint32_t)(kRegMid * kBlock)) {
    resolve_global_regs<kRegMid>(g, slab, need, cnt, sh, o);
  } else {
    if (t < 4) sh.range[t] = ld_agent(&g->range[t]);
    __syncthreads();
    const Refine p = make_refine(sh.range, need, cnt);
    if (!keep) {
      refine<false>(StreamSrc<VEC>{rowp, 0, len, cut, p}, p, sh, o);
    } else if (cnt <= (uint32_t)(kListCap - kLdsCopyWords)) {
      // Pull the list into LDS (direct-to-LDS copy: no registers in flight),
      // rewrite it as composite keys and resolve it there.
      copy_agent_to_lds(slab, cnt, sh.list);
      drain_memory();
      __syncthreads();
      pairs_to_keys(sh, cnt, p);
      refine<true>(KeyListSrc{sh.list, cnt}, p, sh, o);
    } else {
      refine<false>(PairListSrc{slab, cnt, p}, p, sh, o);
    }
  }
  report_bad(!o.flush(n_above, o.k), o.status);
}

// A row shared by w.gsize workgroups; this one holds chunk [w.begin, end).
// EARLY: the predicted-bin vote and early classification are compiled in
// (the variant for tile-sized chunks; elsewhere the code would only cost
// instruction-cache room).
template <bool VEC, bool EARLY>
__device__ __forceinline__ void split_row(const SelectArgs& a, const WorkItem& w, int32_t len, const float* rowp,
                                          const RowOut& o, bool resident, uint32_t (&hk)[kHk], Smem& sh) {
  const int t = threadIdx.x;
  const int32_t begin = w.begin, end = min(w.end, len);
  const uint32_t G = (uint32_t)w.gsize;
  const uint32_t k = (uint32_t)a.k;
  GroupState* g = a.groups + w.group;

  // Only bins at or above this chunk's own k-th bin can hold the row's k-th
  // (bloc). One scan also finds the bin of its T-th largest score (bpre, for
  // the pre-read below) and keeps the prefixes that later give the count
  // above the row's threshold bin. Both stay 0 when the chunk is shorter.
  const uint32_t T = resident ? min(k, 2u * ((k + G - 1u) / G) + 64u) : k;
  uint32_t* cum = sh.outpos;   // free until the extraction stages outputs
  if (t == 0) sh.res[0] = sh.res[3] = 0;
  two_thresholds_raw(sh.lhist, k, T, sh.scratch, cum, &sh.res[0], &sh.res[3]);
  const uint32_t bloc = uni(sh.res[0]);
  // The scores of the chunk that no merged bin counts go to g->arrive, so the
  // merged bins and that count add up to the row length once every
  // workgroup's atomics have landed: there is no separate arrival (and no
  // wait for the atomics before it). The vote below rides on the same
  // check.
  uint32_t merged = 0;
  for (int r = t; r < kBins; r += kBlock) {
    const uint32_t h = sh.lhist[r];
    const uint32_t b = bin_of_raw((uint32_t)r);
    if (h && b >= bloc && b >= kFirstBin && b <= kLastBin) {
      __hip_atomic_fetch_add(&g->hist[r], h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      merged += h;
    }
  }
  const uint32_t chunk = end > begin ? (uint32_t)(end - begin) : 0u;
  // While the other workgroups merge: list the positions at or above the
  // local T-th bin and start reading their scores and block-table entries.
  uint32_t* pre = reinterpret_cast<uint32_t*>(sh.list + kStageCap);
  uint32_t* lfine = reinterpret_cast<uint32_t*>(sh.list + kFineListOff);
  float pv[kPreRegs];
  int32_t ppg[kPreRegs];
  uint32_t n_pre = 0xFFFFFFFFu, bpre = kNotFound;
  // A predicted crowded threshold bin. A chunk whose T-th bin holds many
  // scores while few lie above it expects the row's threshold bin there: it
  // proposes that bin, classifies its pre-read scores against it while the
  // histograms merge, and adds their fine-digit counts to the row early.
  // Every workgroup votes (proposers with v = bin + 1, the others with 0):
  // the proposer count and the sum of v go to the high half of the rest
  // count's word, the sum of v^2 to a word whose low half counts the
  // workgroups, each in one atomic with a part of the completeness check, so
  // the merged histogram's snapshot also holds every vote. The early counts are used only if every proposal
  // equals the row's threshold bin: the count n, the sum and the sum of
  // squares of the proposals then read n, n (b* + 1) and n (b* + 1)^2, which
  // no other set of n proposals gives (see `fine` below).
  bool propose = false;
  uint32_t vote = 0u;
  if (!resident) {
    uint32_t tot_merged;
    block_exclusive_add(merged, sh.scratch, &tot_merged);
    if (t == 0) {
      __hip_atomic_fetch_add(&g->arrive, (uint64_t)(chunk - tot_merged), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if constexpr (EARLY) __hip_atomic_fetch_add(&g->vsq, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    bpre = uni(sh.res[3]);
    const uint64_t pm = interest_mask(hk, cut_of_bin(bpre).vlo);
    // One scan for both the merged count (high half) and the listing offsets
    // (low half): a resident chunk holds at most 32,768 scores, so neither
    // total reaches 2^16.
    static_assert(kTile < (1 << 16), "merged and listed counts share one scan");
    uint32_t tot;
    uint32_t off = block_exclusive_add((merged << 16) | (uint32_t)__popcll(pm), sh.scratch, &tot);
    off &= 0xFFFFu;
    n_pre = uni(tot) & 0xFFFFu;
    // (every score at or above bpre is pre-read, the bin's candidates fit the
    // LDS list below the digit counters, and fewer than k / G lie above it)
    if constexpr (EARLY) {
      const uint32_t lc = uni(sh.lhist[raw_of_bin(bpre)]);
      propose = n_pre <= (uint32_t)kPreCap && lc <= (uint32_t)kFineListOff && lc * G > kFineMin &&
                count_above(sh.lhist, cum, bpre) * G < k;
      vote = propose ? bpre + 1u : 0u;
    }
    if (t == 0) {
      __hip_atomic_fetch_add(&g->arrive,
                             (uint64_t)(chunk - (uni(tot) >> 16)) | ((uint64_t)((uint32_t)propose | (vote << 9)) << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if constexpr (EARLY) {
        __hip_atomic_fetch_add(&g->vsq, (uint64_t)1 | ((uint64_t)(vote * vote) << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        sh.cur_out = 0;
        sh.cur_list = 0;
      }
    }
    if (propose)
      for (int i = t; i < (kFineBins + kFineGroups) / 4; i += kBlock)
        reinterpret_cast<uint4*>(lfine)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (n_pre <= (uint32_t)kPreCap) {
      uint64_t m = pm;
      while (m) {
        const int j = __builtin_ctzll(m);
        m &= m - 1ull;
        pre[off++] = (uint32_t)tile_pos(begin, j >> 2, j & 3);
      }
    }
    __syncthreads();
    if (n_pre <= (uint32_t)kPreCap) {
#pragma unroll
      for (int i = 0; i < kPreRegs; ++i) {
        const uint32_t idx = (uint32_t)(t + i * kBlock);
        const int32_t e = idx < n_pre ? (int32_t)pre[idx] : begin;
        pv[i] = idx < n_pre ? rowp[e] : 0.f;
        ppg[i] = idx < n_pre ? o.page(e) : 0;
      }
    }
  }
  bool spec_bad = false;
  uint32_t* sstaged = reinterpret_cast<uint32_t*>(sh.list + kSpecStageOff);
  uint32_t* sstaged_pg = sstaged + kMaxK;
  if (EARLY && propose) {
    const Cut scut = cut_of_bin(bpre);
    const Refine sf = fine_key_frame(fine_frame(bpre), (uint32_t)len);
    const uint32_t sshift = sf.nb - (uint32_t)kFineBits;
    Range srg;
#pragma unroll
    for (int i = 0; i < kPreRegs; ++i) {
      const uint32_t idx = (uint32_t)(t + i * kBlock);
      if (idx < n_pre)
        classify(
            pv[i], (int32_t)pre[idx], ppg[i], scut, srg,
            [&](int32_t e, int32_t pg) {
              const uint32_t c = atomicAdd(&sh.cur_out, 1u);
              const bool ok = c < (uint32_t)kMaxK;
              if (ok) {
                sstaged[c] = (uint32_t)e;
                sstaged_pg[c] = (uint32_t)pg;
              }
              spec_bad |= !ok;
            },
            [&](uint32_t kk, int32_t e) {
              const uint64_t v = sf.key(kk, e);
              const uint32_t d = min((uint32_t)(v >> sshift), (uint32_t)kFineBins - 1u);
              atomicAdd(&lfine[d], 1u);
              atomicAdd(&lfine[kFineBins + (d >> 6)], 1u);
              const uint32_t c = atomicAdd(&sh.cur_list, 1u);
              const bool ok = c < (uint32_t)kFineListOff;
              if (ok) sh.list[c] = v;
              spec_bad |= !ok;
            });
    }
    __syncthreads();
    merge_fine(lfine, g);
  }
  // Read the merged bins and the rest count until they add up to the row
  // length. Every contribution is a non-negative add, so each value read is
  // at most its final value; a read that sums to the final total therefore
  // read every final value: a consistent snapshot of the merge. Lane t reads
  // the ordered bins 1023 - 2 t and 1022 - 2 t, so the poll's own prefix sum
  // is the count above the lane's bins and the threshold search needs no
  // second scan; the rest count and the vote word go to the last lane, whose
  // bins are the lowest (no bin's prefix includes them).
  static_assert(kBins == 2 * kBlock, "two bins per lane");
  static_assert(offsetof(GroupState, vsq) == offsetof(GroupState, arrive) + 128, "vote word one line past arrive");
  const uint32_t ob0 = (uint32_t)(kBins - 1 - 2 * t), ob1 = ob0 - 1u;
  const uint32_t pr0 = raw_of_bin(ob0), pr1 = raw_of_bin(ob1);
  uint32_t ph0 = 0, ph1 = 0, pcum = 0;
  if (t == 0) sh.res[0] = kNotFound;   // (ordered before the search by the poll's barriers)
  {
    // At most spin_limit polls (uniform); a limit of 0 gives up at once.
    bool ok = false;
    for (uint32_t spins = 0; spins < a.spin_limit; ++spins) {
      ph0 = ld_agent(&g->hist[pr0]);
      ph1 = ld_agent(&g->hist[pr1]);
      const bool last = t == kBlock - 1;
      const uint64_t va = last ? ld_agent(&g->arrive) : (uint64_t)0;
      const uint64_t vq = EARLY && last ? ld_agent(&g->vsq) : (uint64_t)0;
      if (last) {
        sh.pl_red2[0] = (uint32_t)(va >> 32);
        sh.pl_red2[1] = (uint32_t)(vq >> 32);
      }
      uint32_t tot;
      pcum = block_exclusive_add(ph0 + ph1 + (uint32_t)va + (uint32_t)vq, sh.scratch, &tot);
      if (uni(tot) == (uint32_t)len + (EARLY ? G : 0u)) {   // (the rest count, then one per workgroup)
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) {
      if (t == 0) atomicOr(a.status, TOPK_DEVICE_SPIN_TIMEOUT);
      return;
    }
  }
  // Bins at or above the largest chunk threshold are complete, and the row's
  // threshold bin lies there, so the count from the top is exact (NaN bins
  // are never merged and read 0). Not found only with NaN inputs; the
  // workgroup then skips its emission but still takes part in the arrival
  // count so the row's state is reset.
  if (pcum < k && k <= pcum + ph0 + ph1) {
    const bool hi = k <= pcum + ph0;
    sh.res[0] = hi ? ob0 : ob1;
    sh.res[1] = hi ? pcum : pcum + ph0;
    sh.res[2] = hi ? ph0 : ph1;
  }
  __syncthreads();
  const uint32_t r0 = uni(sh.res[0]);
  const bool found = r0 != kNotFound;
  if (!found && t == 0) atomicOr(a.status, TOPK_DEVICE_INTERNAL);
  const uint32_t bstar = found ? r0 : kLastBin;
  const uint32_t n_above = found ? uni(sh.res[1]) : 0u, cnt = found ? uni(sh.res[2]) : 0u;
  const Cut cut = cut_of_bin(bstar);
  const uint32_t local_above = found ? count_above(sh.lhist, cum, bstar) : 0u;
  const uint32_t local_cnt = found ? uni(sh.lhist[raw_of_bin(bstar)]) : 0u;
  const bool keep = found && (int64_t)cnt <= a.cand_cap;
  const bool stage = keep && local_cnt <= (uint32_t)kStageCap;   // candidates staged in LDS
  // A large threshold bin (uniform across the row's workgroups): its
  // candidates are also counted by fine digit, in LDS when the staged list
  // leaves room for the counters, else straight into the row's global digit
  // histogram. With a predicted bin, only if the prediction holds: the
  // digit histogram then already holds the early counts, and the workgroups
  // that made them skip their classification (pre_done); a wrong prediction
  // leaves stray counts, so the row takes the path without digit counts.
  const uint32_t n_prop = EARLY ? uni(sh.pl_red2[0]) & 511u : 0u;
  const uint64_t b1 = (uint64_t)bstar + 1u;
  const bool agree = !EARLY || ((uint64_t)(uni(sh.pl_red2[0]) >> 9) == n_prop * b1 &&
                                (uint64_t)uni(sh.pl_red2[1]) == n_prop * b1 * b1);
  const bool fine = keep && cnt > kFineMin && cnt <= kFineMaxCand && agree;   // (n_prop = 0 agrees)
  const bool pre_done = EARLY && propose && fine;   // (then this workgroup's proposal is b*)
  const bool fine_lds = local_cnt <= (uint32_t)kFineListOff;
  const Refine pf = fine_key_frame(fine_frame(bstar), (uint32_t)len);
  const uint32_t dshift = pf.nb - (uint32_t)kFineBits;
  // This workgroup's output and candidate offsets in the row; their round
  // trips overlap the re-reads of the extraction below.
  // Thread 0 uses the atomics' results only after the extraction (nothing
  // before that barrier may depend on them, or the whole workgroup would wait
  // for the round trip); only the rare unstaged case, candidates written
  // straight to global memory, needs its base first.
  uint32_t base_out = 0, base_cand = 0;
  if (t == 0 && !pre_done) {
    sh.cur_out = 0;
    sh.cur_list = 0;
    sh.range[0] = sh.range[1] = sh.range[2] = sh.range[3] = 0;
    // The zero offset hides that one lane runs this: offered a uniform
    // address, the compiler turns each fetch-add into its wave-aggregated
    // form, which reads the result back at once and so waits here.
    const uint32_t z = opaque_zero();
    if (local_above && !fine)
      base_out = __hip_atomic_fetch_add(&g->emit + z, local_above, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (keep && local_cnt && !fine)
      base_cand = __hip_atomic_fetch_add(&g->cand + z, local_cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (fine && !pre_done) {   // digit counters (every wave has read its local bins above)
    if (fine_lds)
      for (int i = t; i < (kFineBins + kFineGroups) / 4; i += kBlock)
        reinterpret_cast<uint4*>(lfine)[i] = make_uint4(0u, 0u, 0u, 0u);
    else if (t < kFineGroups)
      sh.lhist[t] = 0u;
    __syncthreads();
  }
  if (keep && !stage) {
    if (t == 0) sh.cur_list = base_cand;
    __syncthreads();
  }
  uint64_t* slab = a.cand + (int64_t)w.group * a.cand_cap;
  uint32_t* staged = sh.rhist;     // positions above the threshold bin (< k of them)
  uint32_t* staged_pg = sh.outpos; // and their block-table entries
  Range rg;
  bool bad = false;
  auto on_above = [&](int32_t e, int32_t pg) {
    const uint32_t c = atomicAdd(&sh.cur_out, 1u);
    const bool ok = c < (uint32_t)kMaxK;
    if (ok) {
      staged[c] = (uint32_t)e;
      staged_pg[c] = (uint32_t)pg;
    }
    bad |= !ok;
  };
  auto on_cand = [&](uint32_t kk, int32_t e) {
    if (!keep) return;
    // fine rows store the fine-frame composite key, others (key32, position)
    const uint64_t v = fine ? pf.key(kk, e) : ((uint64_t)kk << 32) | (uint32_t)e;
    if (fine) {
      const uint32_t d = min((uint32_t)(v >> dshift), (uint32_t)kFineBins - 1u);
      if (fine_lds) {
        // (the first increment of a digit appends it: a uniform-address
        // append the compiler aggregates per wave)
        atomicAdd(&lfine[d], 1u);
        atomicAdd(&lfine[kFineBins + (d >> 6)], 1u);
      } else {
        __hip_atomic_fetch_add(&g->fine[d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomicAdd(&sh.lhist[d >> 6], 1u);
      }
    }
    const uint32_t c = atomicAdd(&sh.cur_list, 1u);
    const bool ok = stage ? c < (uint32_t)kStageCap : (int64_t)c < a.cand_cap;
    if (ok && stage) sh.list[c] = v;
    if (ok && !stage) st_agent(slab + c, v);
    bad |= !ok;
  };
  if (found && !pre_done) {
    if (resident && n_pre <= (uint32_t)kPreCap && bstar >= bpre) {
      // Every position at or above the row's threshold bin was pre-read.
#pragma unroll
      for (int i = 0; i < kPreRegs; ++i) {
        const uint32_t idx = (uint32_t)(t + i * kBlock);
        if (idx < n_pre) classify(pv[i], (int32_t)pre[idx], ppg[i], cut, rg, on_above, on_cand);
      }
    } else if (resident) {
      load_pack<VEC>(rowp, begin, end, hk);   // (the tile is not held across the wait)
      extract(interest_mask(hk, cut.vlo), begin, rowp, cut.vhi, rg, on_above, on_cand, &o);
    } else {
      for (int32_t base = begin; base < end; base += kTile) {
        load_pack<VEC>(rowp, base, end, hk);
        extract(interest_mask(hk, cut.vlo), base, rowp, cut.vhi, rg, on_above, on_cand, &o);
      }
    }
  }
  if (fine) {
    if (pre_done)
      fine_tail<VEC>(a, g, slab, len, G, k, n_above, cnt, local_above, kFineMerged, pf, sh, o, bad || spec_bad,
                     sstaged, sstaged_pg, (uint32_t)kSpecStageOff);
    else
      fine_tail<VEC>(a, g, slab, len, G, k, n_above, cnt, local_above, fine_lds ? kFineInLds : kFineGlobal, pf, sh,
                     o, bad, sh.rhist, sh.outpos, (uint32_t)kStageCap);
    return;
  }
  merge_range(rg, sh);
  __syncthreads();
  if (t == 0) {
    sh.bcast[0] = base_out;
    sh.bcast[1] = base_cand;
    if (local_cnt) {
      __hip_atomic_fetch_max(&g->range[0], sh.range[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(&g->range[1], sh.range[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(&g->range[2], sh.range[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(&g->range[3], sh.range[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  // Staged candidates, then outputs, leave in consecutive, coalesced stores.
  // Only the candidates must have landed before the arrival count (the last
  // workgroup reads them); no workgroup reads the outputs, so waves 1 to 7
  // store them while wave 0 makes the round trip of `done`.
  const uint32_t bo = uni(sh.bcast[0]), bc = uni(sh.bcast[1]);
  const uint32_t n_out = min(uni(sh.cur_out), (uint32_t)kMaxK);
  if (stage) {
    const uint32_t n_c = min(uni(sh.cur_list), (uint32_t)kStageCap);
    for (uint32_t i = t; i < n_c; i += kBlock) {
      const bool ok = (int64_t)(bc + i) < a.cand_cap;
      if (ok) st_agent(slab + bc + i, sh.list[i]);
      bad |= !ok;
    }
  }
  drain_memory();
  __syncthreads();
  if (t == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&g->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = prev == G - 1;
  } else if (t >= kWave) {
    for (uint32_t i = t - kWave; i < n_out; i += kBlock - kWave)
      bad |= !o.store_page(bo + i, (int32_t)staged[i], (int32_t)staged_pg[i]);
  }
  report_bad(bad, a.status);
  __syncthreads();
  if (!uni(sh.flag)) return;
  // Last workgroup of the row: resolve the threshold bin, then leave the
  // row's state zeroed for the next call.
  if (found) resolve_split<VEC>(a, g, slab, keep, len, rowp, cut, k - n_above, cnt, n_above, sh, o);
  if (EARLY && n_prop) {   // (early counts of a predicted bin)
    uint64_t* fg = reinterpret_cast<uint64_t*>(g->fine);
    for (int i = t; i < kFineBins / 2; i += kBlock) st_agent(fg + i, (uint64_t)0);
    if (t < kFineGroups) st_agent(&g->fine_c[t], 0u);
  }
  for (int r = t; r < kBins; r += kBlock) st_agent(&g->hist[r], 0u);
  if (t < 4) st_agent(&g->range[t], 0u);
  if (t == 0) {
    st_agent(&g->arrive, (uint64_t)0);
    st_agent(&g->vsq, (uint64_t)0);
    st_agent(&g->emit, 0u);
    st_agent(&g->cand, 0u);
    st_agent(&g->done, 0u);
  }
}

// The packed register tile parked in the upper half of the LDS list (lane
// t's register i at word i * kBlock + t), clear of the histogram copies.
__device__ __forceinline__ uint32_t* parked_tile(Smem& sh) {
  return reinterpret_cast<uint32_t*>(sh.list + kListCap / 2);
}
static_assert(kHk * kBlock * 4 <= kListCap / 2 * 8, "a parked tile fits in half the LDS list");
static_assert(kBins * kHistCopies * 4 <= kListCap / 2 * 8, "histogram copies fit below a parked tile");

// parked: this item's register tile is already in LDS (parked_tile).
// STREAM: items longer than one register tile can occur (otherwise their code
// is left out, which keeps it from weighing on the resident path's registers).
// PQ: vector groups a parked tile holds (the rest of it is NaN padding).
template <bool VEC, bool STREAM, bool EARLY, int PQ>
__device__ __forceinline__ void process_item(const SelectArgs& a, const WorkItem& item, Smem& sh, bool parked = false) {
  const int t = threadIdx.x;
  // (every field is uniform: held in scalar registers)
  WorkItem w;
  w.row = (int32_t)uni((uint32_t)item.row);
  w.begin = (int32_t)uni((uint32_t)item.begin);
  w.end = (int32_t)uni((uint32_t)item.end);
  w.group = (int32_t)uni((uint32_t)item.group);
  w.gsize = (int32_t)uni((uint32_t)item.gsize);
  w.len = (int32_t)uni((uint32_t)item.len);
  w.pad[0] = w.pad[1] = 0;
  const int row = w.row;
  const int32_t len = w.len;   // planned from the same lengths (one dependent load fewer)
  if (len < 0 || (int64_t)len > a.max_len) {
    if (t == 0) atomicOr(a.status, TOPK_DEVICE_BAD_LENGTH);
    return;
  }
  RowOut o;
  o.slots = a.out_slots + (int64_t)row * a.out_stride;
  o.idx = a.out_idx ? a.out_idx + (int64_t)row * a.out_stride : nullptr;
  o.table = a.table + (int64_t)row * a.table_stride;
  o.ps = a.page_size;
  o.shift = a.page_shift;
  o.k = (uint32_t)a.k;
  o.len = (uint32_t)len;
  o.status = a.status;
  o.stage = sh.outpos;
  if (len <= a.k) {  // every valid position is selected; pad with -1
    if (w.begin == 0) {
      for (int j = t; j < a.k; j += kBlock) {
        if (j < len) {
          o.store((uint32_t)j, j);
        } else {
          o.slots[j] = -1;
          if (o.idx) o.idx[j] = -1;
        }
      }
    }
    return;
  }
  const float* rowp = a.scores + (int64_t)row * a.stride;
  const int32_t begin = w.begin, end = min(w.end, len);
  bool resident = end - begin <= kTile;
  if constexpr (!STREAM) {
    if (!resident) {   // excluded by the host's choice of variant; never silently
      if (t == 0) atomicOr(a.status, TOPK_DEVICE_INTERNAL);
      return;
    }
    resident = true;
  }
  uint32_t hk[kHk];
  uint32_t* hc = reinterpret_cast<uint32_t*>(sh.list);   // free until the extraction
  if (!parked) {   // (a parked tile's histogram is already in the copies)
    hist_copies_clear(hc);
    __syncthreads();
  }
  if (resident) {
    if (parked) {
      const uint32_t* pt = parked_tile(sh);
#pragma unroll
      for (int i = 0; i < kHk; ++i) hk[i] = i < 2 * PQ ? pt[i * kBlock + t] : kHalfNaN2;
    } else {
      float4 x[kEpt / 4];
      load_raw<VEC>(rowp, begin, end, x);
      pack_hist(x, begin, end, hk, hc);
    }
  } else {
    // Streamed in half tiles: the next half's loads are in flight while this
    // one is binned.
    constexpr int kHalf = kEpt / 8;   // dwordx4 per lane per step
    constexpr int32_t kStep = kHalf * kBlock * 4;
    float4 xa[kHalf];
    load_vecs<VEC, kHalf>(rowp, begin, end, xa);
    for (int32_t base = begin; base < end; base += kStep) {
      float4 xb[kHalf];
      if (base + kStep < end) load_vecs<VEC, kHalf>(rowp, base + kStep, end, xb);
      hist_vecs<kHalf>(xa, hc, base, end);
#pragma unroll
      for (int q = 0; q < kHalf; ++q) xa[q] = xb[q];
    }
  }
  __syncthreads();
  hist_copies_sum(hc, sh.lhist);
  __syncthreads();
  if (w.group < 0) owned_row<VEC, STREAM>(a, len, rowp, o, resident, hk, sh);
  else split_row<VEC, EARLY>(a, w, len, rowp, o, resident, hk, sh);
}

// In-kernel planning for small batches: thread t holds row t. Every
// workgroup computes the same split counts and item offsets as
// topk_plan_kernel (the same split_of) and writes the items that fall to it
// (item it goes to workgroup it % grid, as in the plan-buffer loop) into LDS.
// Returns the number of items, or -1 if the plan would not fit.

__device__ __forceinline__ PlanArgs plan_args_of(const SelectArgs& a) {
  PlanArgs p;
  p.lengths = a.lengths;
  p.num_rows = a.num_rows;
  p.k = a.k;
  p.grid = (int32_t)gridDim.x;
  p.max_groups = a.max_groups;
  p.max_items = 0;
  p.force_path = a.force_path;
  p.wg_per_row = a.wg_per_row;
  p.min_chunk = a.min_chunk;
  p.max_len = a.max_len;
  p.header = nullptr;
  p.items = nullptr;
  return p;
}

__device__ __forceinline__ int plan_here(const SelectArgs& a, Smem& sh, int32_t len) {
  const int t = threadIdx.x;
  const int R = a.num_rows;
  // narrow (uniform): at most one wave of rows, and `len` is then row
  // lane()'s length in every wave, so each wave reduces and scans on its own
  // (cross-lane moves, no LDS exchange, no barrier). Otherwise `len` is row
  // t's and the waves combine through LDS.
  const bool narrow = R <= kWave;
  const int r = t & (narrow ? kWave - 1 : kBlock - 1);
  const bool longer = r < R && len > split_floor(plan_args_of(a));
  // Wave sums (lengths < 2^31: 64 halves of 16 and 15 bits fit a word).
  const uint32_t lo = wave_sum_u32(longer ? (uint32_t)len & 0xFFFFu : 0u);
  const uint32_t hi = wave_sum_u32(longer ? (uint32_t)len >> 16 : 0u);
  uint64_t total = ((uint64_t)hi << 16) + lo;
  int32_t n_long = (int32_t)__popcll(__ballot(longer));
  uint32_t tiles = wave_sum_u32(longer ? (uint32_t)tiles_of(len) : 0u);
  if (!narrow) {   // combine the waves' sums
    if (lane() == 0) {
      sh.pl_red[t >> 6] = total | ((uint64_t)n_long << 40);   // rows < 2^23
      sh.pl_red2[t >> 6] = tiles;
    }
    __syncthreads();
    uint64_t packed = 0;
    tiles = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      packed += sh.pl_red[i];
      tiles += sh.pl_red2[i];
    }
    total = packed & ((1ull << 40) - 1);
    n_long = (int32_t)(packed >> 40);
  }
  int64_t c;
  const int g = r < R ? split_of(len, plan_args_of(a), total, n_long, tiles, &c) : 0;
  // One scan of three packed counts: split items (12 bits: at most the
  // grid, which the host keeps below 4096 for this path), split rows and
  // whole rows (10 bits each: at most kInKernelPlanRows).
  const uint32_t packed_n = (g > 1 ? (uint32_t)g | (1u << 12) : 0u) | (g == 1 ? 1u << 22 : 0u);
  uint32_t packed_tot, packed_off;
  if (narrow) {
    const uint32_t inc = wave_inclusive_add(packed_n);
    packed_off = inc - packed_n;
    packed_tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
  } else {
    packed_off = block_exclusive_add(packed_n, sh.scratch, &packed_tot);
  }
  // The items are written by threads t < R, which hold row t either way
  // (narrow: R <= kWave puts them all in wave 0, where r == t).
  const uint32_t off_m = packed_off & 0xFFFu, off_g = (packed_off >> 12) & 0x3FFu, off_s = packed_off >> 22;
  const uint32_t tot_m = packed_tot & 0xFFFu, tot_g = (packed_tot >> 12) & 0x3FFu, tot_s = packed_tot >> 22;
  const int G = (int)gridDim.x, B = (int)blockIdx.x;
  const int num_items = (int)(tot_m + tot_s);
  if (t < R && g > 1) {
    // the one split item of this row that falls to this workgroup, if any
    const int j = B - (int)off_m;
    if (j >= 0 && j < g) {
      const int64_t e = (int64_t)(j + 1) * c;
      WorkItem w;
      w.row = t;
      w.begin = (int32_t)(j * c);
      w.end = (int32_t)(e < len ? e : len);
      w.group = (int32_t)off_g;
      w.gsize = g;
      w.len = len;
      w.pad[0] = w.pad[1] = 0;
      sh.pl_items[0] = w;
    }
  } else if (t < R) {
    const int it = (int)tot_m + (int)off_s;
    const int m = (it - B) / G;
    if (it % G == B && m < kMaxLocalItems) {
      WorkItem w;
      w.row = t;
      w.begin = 0;
      w.end = len;
      w.group = -1;
      w.gsize = 1;
      w.len = (len < 0 || (int64_t)len > a.max_len) ? -1 : len;
      w.pad[0] = w.pad[1] = 0;
      sh.pl_items[m] = w;
    }
  }
  __syncthreads();
  // (uniform: workgroup 0 takes the most items)
  const bool fits = tot_m <= (uint32_t)G && (int)tot_g <= a.max_groups && (num_items - 1) / G < kMaxLocalItems;
  return fits ? num_items : -1;
}

// In-kernel planning with a guessed first tile. Each workgroup starts
// loading the tile it would get if every row had max_len scores, before the
// lengths arrive, then plans; the loads are used when the real plan gives the
// same chunk (every batch of equal lengths), and the tile is then packed,
// binned and parked in LDS. Returns whether it was; num_items as plan_here.
// OVERLAP > 0: the lengths are requested first and the tile (its first
// OVERLAP vector groups, which hold the guessed chunk) goes through a
// buffer resource (no per-lane branches), so the planning waits for the
// lengths only and runs while the tile arrives. Without it, the tile is
// converted as it arrives and the planning follows.
template <bool VEC, int OVERLAP>
__device__ __forceinline__ bool guess_and_plan(const SelectArgs& a, Smem& sh, int& num_items) {
  int32_t len_t = 0;
  if constexpr (OVERLAP > 0) {
    // (loads complete in order: waiting for the length does not wait for the tile)
    const int r = (int)threadIdx.x & (a.num_rows <= kWave ? kWave - 1 : kBlock - 1);   // as plan_here reads it
    len_t = r < a.num_rows ? a.lengths[r] : 0;
    asm volatile("" ::: "memory");
  }
  float4 x[kEpt / 4];
  int32_t srow = -1, sbeg = 0, send = 0;
  // (uniform across the workgroup: every value below derives from kernel
  // arguments and blockIdx)
  {
    const int32_t L = (int32_t)a.max_len;
    const int g = a.guess_groups;       // the planner's split of a max_len row,
    const int64_t c = a.guess_chunk;    // worked out by the host
    const int B = (int)blockIdx.x;
    if (g > 1 && B < a.num_rows * g) {
      srow = B / g;
      sbeg = (int32_t)((B % g) * c);
      send = (int32_t)min((int64_t)sbeg + c, (int64_t)L);
    } else if (g <= 1 && L > a.k && B < a.num_rows) {
      srow = B;
      send = L;
    }
    if constexpr (OVERLAP > 0) {
      if (srow < 0 || send - sbeg > OVERLAP * kBlock * 4) {   // no guess that fits: nothing is read
        srow = -1;
        sbeg = send = 0;
      }
      load_raw_buffer<VEC, OVERLAP>(a.scores + (int64_t)max(srow, 0) * a.stride, sbeg, send, x);
    } else {
      if (srow >= 0 && send - sbeg <= kTile) load_raw<VEC>(a.scores + (int64_t)srow * a.stride, sbeg, send, x);
      else srow = -1;
    }
  }
  // (the barriers of the planning order this clear before any histogram add)
  if (srow >= 0) hist_copies_clear(reinterpret_cast<uint32_t*>(sh.list));
  if constexpr (OVERLAP == 0) {
    const int r = (int)threadIdx.x & (a.num_rows <= kWave ? kWave - 1 : kBlock - 1);   // as plan_here reads it
    len_t = r < a.num_rows ? a.lengths[r] : 0;
  }
  num_items = plan_here(a, sh, len_t);
  if constexpr (OVERLAP > 0) {
    // Keep the tile's first use here: the compiler would otherwise convert
    // each vector as it arrives, ahead of the planning, and the planning
    // would then wait for the whole tile.
#pragma unroll
    for (int q = 0; q < OVERLAP; ++q) asm volatile("" : "+v"(x[q].x), "+v"(x[q].y), "+v"(x[q].z), "+v"(x[q].w));
  }
  if (num_items < 0) return false;
  // Park the tile if the real plan gave the guessed chunk (the same row and
  // start, ending no later; positions past the real end become NaN),
  // binning each vector as it arrives.
  bool parked = false;
  if ((int)blockIdx.x < num_items && srow >= 0) {
    const WorkItem w0 = sh.pl_items[0];
    const int32_t end0 = min(w0.end, w0.len);
    parked = w0.row == srow && w0.begin == sbeg && end0 <= send && w0.len > a.k && (int64_t)w0.len <= a.max_len;
    if (parked) {
      uint32_t hk[kHk];
      // (OVERLAP > 0: a guessed chunk spans at most OVERLAP vector groups)
      pack_hist<(OVERLAP > 0 ? OVERLAP : kEpt / 4)>(x, sbeg, end0, hk, reinterpret_cast<uint32_t*>(sh.list));
      // (only the vector groups the guess spans: the rest are NaN padding,
      // which the unparking rebuilds)
      uint32_t* pt = parked_tile(sh);
#pragma unroll
      for (int i = 0; i < 2 * (OVERLAP > 0 ? OVERLAP : kEpt / 4); ++i) pt[i * kBlock + threadIdx.x] = hk[i];
    }
  }
  return parked;
}

// OVERLAP > 0: the in-kernel planning overlaps the loads of the guessed
// tile's first OVERLAP vector groups (chosen by the host: 16 for guessed
// tiles of at least half a tile, 4 for those of at most 8,192 scores; in
// between, the conditional loads skip empty vector groups, which is worth
// more than the overlap).
template <bool VEC, bool STREAM, int OVERLAP>
__global__ void __launch_bounds__(kBlock) topk_select_kernel(SelectArgs a) {
  __shared__ Smem sh;
  int num_items;
  bool parked = false;
  if (a.plan) {
    // The first item is fetched together with the header and staged in LDS
    // (the plan buffer always holds at least gridDim.x items, so the read
    // stays in bounds; the item is used only if the header says it exists).
    if (threadIdx.x == 0) sh.pl_items[0] = a.items[blockIdx.x];
    const PlanHeader h = *a.plan;
    if (h.magic != kPlanMagic || h.k != a.k || h.grid != (int)gridDim.x || h.num_rows > a.num_rows) {
      if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(a.status, TOPK_DEVICE_PLAN_MISMATCH);
      return;
    }
    num_items = h.num_items;
  } else {
    parked = guess_and_plan<VEC, OVERLAP>(a, sh, num_items);
    if (num_items < 0) {
      if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(a.status, TOPK_DEVICE_PLAN_MISMATCH);
      return;
    }
  }
  for (int it = blockIdx.x; it < num_items; it += gridDim.x) {
    // Items are read from LDS: a plan-buffer item is staged in slot 0 (the
    // barrier after the previous item keeps it from being overwritten early).
    int slot = 0;
    if (a.plan) {
      if (threadIdx.x == 0 && it != (int)blockIdx.x) sh.pl_items[0] = a.items[it];
      __syncthreads();
    } else {
      slot = (it - (int)blockIdx.x) / (int)gridDim.x;
    }
    process_item<VEC, STREAM, (OVERLAP >= kEpt / 4), (OVERLAP > 0 ? OVERLAP : kEpt / 4)>(
        a, sh.pl_items[slot], sh, parked && it == (int)blockIdx.x);
    __syncthreads();
  }
}

__global__ void topk_fill_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// The selection kernel's own binning and FP32 key, element by element.
__global__ void topk_debug_keys_kernel(const float* x, int64_t n, uint32_t* bin, uint32_t* k32) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float v = x[i];
    if (bin) bin[i] = bin_of_raw((to_half2(v, v) >> 6) & 0x3FFu);
    if (k32) k32[i] = key32_of(v);
  }
}

// The selection kernel's coarse histogram and threshold bin of each row, with
// its own binning (pack_hist into interleaved copies, hist_copies_sum) and its
// own threshold scan (find_threshold_raw). One workgroup per row; rows are
// read in whole tiles with per-element loads (any alignment). Writes
// hist[r][b] for ordered bins b (NaN-only bins included) and, for rows longer
// than k, res[r] = {b*, scores above b*, scores in b*}; shorter rows get
// {kNotFound, 0, 0}.
struct __align__(16) DebugSmem {
  uint32_t hc[kBins * kHistCopies];
  uint32_t h[kBins];
  uint32_t scratch[kWaves];
  uint32_t res[4];
};

__global__ void __launch_bounds__(kBlock) topk_debug_hist_kernel(const float* scores, int64_t stride,
                                                                  const int32_t* lengths, int32_t k,
                                                                  uint32_t* hist, uint32_t* res) {
  __shared__ DebugSmem sh;
  const int r = blockIdx.x;
  const int32_t len = lengths[r];
  const float* rowp = scores + (int64_t)r * stride;
  hist_copies_clear(sh.hc);
  __syncthreads();
  for (int32_t base = 0; base < len; base += kTile) {
    float4 x[kEpt / 4];
    uint32_t hk[kHk];
    load_raw<false>(rowp, base, len, x);
    pack_hist(x, base, len, hk, sh.hc);
  }
  __syncthreads();
  hist_copies_sum(sh.hc, sh.h);
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kBlock) hist[(int64_t)r * kBins + b] = sh.h[raw_of_bin((uint32_t)b)];
  if (threadIdx.x == 0) sh.res[0] = kNotFound, sh.res[1] = sh.res[2] = 0;
  __syncthreads();
  if (len > k) find_threshold_raw(sh.h, (uint32_t)k, sh.scratch, sh.res);
  if (threadIdx.x < 3) res[(int64_t)r * 3 + threadIdx.x] = sh.res[threadIdx.x];
}

// Streaming-read ceiling: each workgroup reads its contiguous share of x with
// the selection kernel's load pattern (lane t takes vector q * kBlock + t,
// 16 vectors in flight) and writes one partial sum.
constexpr int kStreamReadGroups = 256;
__global__ void __launch_bounds__(kBlock) topk_stream_read_kernel(const float4* x, int64_t nvec, int64_t per_group,
                                                                  float* out) {
  __shared__ float part[kWaves];
  const int64_t begin = (int64_t)blockIdx.x * per_group;
  const int64_t end = min(begin + per_group, nvec);
  float acc = 0.f;
  for (int64_t base = begin; base < end; base += (int64_t)kEpt / 4 * kBlock) {
    float4 v[kEpt / 4];
#pragma unroll
    for (int q = 0; q < kEpt / 4; ++q) {
      const int64_t i = base + (int64_t)q * kBlock + threadIdx.x;
      v[q] = i < end ? x[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < kEpt / 4; ++q) acc += (v[q].x + v[q].y) + (v[q].z + v[q].w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane() == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += part[w];
    out[blockIdx.x] = sum;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI in topk_api.hip).
// ---------------------------------------------------------------------------
hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_plan_kernel, dim3(1), dim3(kPlanBlock), 0, s, a);
  return hipGetLastError();
}

// With events, they record the dispatch's own start and end (the same
// interval a kernel trace reports), not the stream position around it.
template <bool VEC, bool STREAM, int OVERLAP>
void launch_select_t(const SelectArgs& a, int grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  void (*kernel)(SelectArgs) = topk_select_kernel<VEC, STREAM, OVERLAP>;
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), 0, s, start, stop, 0, a);
  else
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), 0, s, a);
}

hipError_t launch_select(const SelectArgs& a, int grid, bool vec, bool stream_items, int overlap, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  if (vec && stream_items) {
    if (overlap == 16) launch_select_t<true, true, 16>(a, grid, s, start, stop);
    else if (overlap == 4) launch_select_t<true, true, 4>(a, grid, s, start, stop);
    else launch_select_t<true, true, 0>(a, grid, s, start, stop);
  } else if (vec) {
    if (overlap == 16) launch_select_t<true, false, 16>(a, grid, s, start, stop);
    else if (overlap == 4) launch_select_t<true, false, 4>(a, grid, s, start, stop);
    else launch_select_t<true, false, 0>(a, grid, s, start, stop);
  } else if (stream_items) {
    launch_select_t<false, true, 0>(a, grid, s, start, stop);
  } else {
    launch_select_t<false, false, 0>(a, grid, s, start, stop);
  }
  return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(topk_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, n);
  return hipGetLastError();
}

hipError_t launch_debug_keys(const float* x, int64_t n, uint32_t* bin, uint32_t* k32, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(topk_debug_keys_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n, bin, k32);
  return hipGetLastError();
}

hipError_t launch_stream_read(const float* x, int64_t n, float* out, hipStream_t s, hipEvent_t start,
                              hipEvent_t stop) {
  const int64_t nvec = n / 4;
  const int64_t per_group = (nvec + kStreamReadGroups - 1) / kStreamReadGroups;
  const float4* xv = reinterpret_cast<const float4*>(x);
  if (start && stop)
    hipExtLaunchKernelGGL(topk_stream_read_kernel, dim3(kStreamReadGroups), dim3(kBlock), 0, s, start, stop, 0, xv,
                          nvec, per_group, out);
  else
    hipLaunchKernelGGL(topk_stream_read_kernel, dim3(kStreamReadGroups), dim3(kBlock), 0, s, xv, nvec, per_group,
                       out);
  return hipGetLastError();
}

int stream_read_groups() { return kStreamReadGroups; }

hipError_t launch_debug_hist(const float* scores, int64_t stride, const int32_t* lengths, int32_t rows, int32_t k,
                             uint32_t* hist, uint32_t* res, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_debug_hist_kernel, dim3(rows), dim3(kBlock), 0, s, scores, stride, lengths, k, hist, res);
  return hipGetLastError();
}

hipError_t select_occupancy(int* per_cu) {
  int a = 0, b = 0;
  const void* kernels[8] = {(const void*)topk_select_kernel<true, true, 0>,
                            (const void*)topk_select_kernel<true, false, 0>,
                            (const void*)topk_select_kernel<true, true, 16>,
                            (const void*)topk_select_kernel<true, false, 16>,
                            (const void*)topk_select_kernel<true, true, 4>,
                            (const void*)topk_select_kernel<true, false, 4>,
                            (const void*)topk_select_kernel<false, true, 0>,
                            (const void*)topk_select_kernel<false, false, 0>};
  int best = 1 << 30;
  for (const void* f : kernels) {
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, f, kBlock, 0);
    if (e != hipSuccess) return e;
    best = a < best ? a : best;
  }
  (void)b;
  *per_cu = best;
  return hipSuccess;
}

}  // namespace satopk
