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

#include "sparse_topk.h"
#include "topk_device.hpp"
#include "topk_layout.hpp"

namespace satopk {

// ---------------------------------------------------------------------------
// Planning kernel: one workgroup reads the device lengths and writes the plan.
// ---------------------------------------------------------------------------
constexpr int kPlanBlock = 1024;

__device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
__device__ __forceinline__ int64_t round_up64(int64_t a, int64_t b) { return ceil_div64(a, b) * b; }

// Workgroups a row gets for target chunk `chunk`; 1 = the row stays whole.
// `chunk_out` receives the aligned chunk length actually used.
__device__ __forceinline__ int split_of(int32_t len, int32_t k, int64_t chunk, bool force_split,
                                        int32_t fixed_g, int64_t* chunk_out) {
  *chunk_out = len;
  if (len <= k) return 1;
  int64_t g = fixed_g > 0 ? fixed_g : ceil_div64(len, chunk);
  if (force_split && g < 2) g = 2;
  if (g < 2) return 1;
  const int64_t c = round_up64(ceil_div64(len, g), kChunkAlign);
  g = ceil_div64(len, c);
  if (g < 2) return 1;
  *chunk_out = c;
  return (int)g;
}

__global__ void __launch_bounds__(kPlanBlock) topk_plan_kernel(PlanArgs a) {
  __shared__ unsigned long long s_total;
  __shared__ int s_items, s_groups, s_ok;
  __shared__ uint32_t s_scan[kPlanBlock / 64];
  __shared__ int s_carry_multi, s_carry_groups, s_carry_single;
  const int t = threadIdx.x;
  const bool no_split = a.force_path == TOPK_PATH_REGISTER || a.force_path == TOPK_PATH_SINGLE;
  const bool force_split = a.force_path == TOPK_PATH_MULTI;

  if (t == 0) s_total = 0;
  __syncthreads();
  unsigned long long mine = 0;
  for (int r = t; r < a.num_rows; r += kPlanBlock) {
    const int32_t len = a.lengths[r];
    if (len > a.k) mine += (unsigned long long)len;
  }
  atomicAdd(&s_total, mine);
  __syncthreads();

  // Target chunk: spread the batch's work over the persistent grid, then grow
  // the chunk until the split rows' items fit in one round of the grid.
  int64_t chunk = round_up64((int64_t)a.min_chunk > 0 ? a.min_chunk : kDefaultMinChunk, kChunkAlign);
  const int64_t even = round_up64(ceil_div64((int64_t)s_total, a.grid > 0 ? a.grid : 1), kChunkAlign);
  if (even > chunk) chunk = even;
  if (no_split) chunk = (int64_t)1 << 40;
  for (int iter = 0; iter < 128; ++iter) {
    if (t == 0) { s_items = 0; s_groups = 0; }
    __syncthreads();
    int items = 0, groups = 0;
    for (int r = t; r < a.num_rows; r += kPlanBlock) {
      int64_t c;
      const int g = split_of(a.lengths[r], a.k, chunk, force_split, a.wg_per_row, &c);
      if (g > 1) { items += g; groups += 1; }
    }
    atomicAdd(&s_items, items);
    atomicAdd(&s_groups, groups);
    __syncthreads();
    const bool fits = s_items <= a.grid && s_groups <= a.max_groups;
    __syncthreads();
    if (fits || a.wg_per_row > 0) break;
    chunk = round_up64(chunk + chunk / 4 + kChunkAlign, kChunkAlign);
  }
  const int total_multi = s_items;
  if (t == 0) {
    s_ok = (s_items <= a.grid && s_groups <= a.max_groups) ? 1 : 0;
    s_carry_multi = 0;
    s_carry_groups = 0;
    s_carry_single = 0;
  }
  __syncthreads();
  if (!s_ok) {  // only reachable with a fixed wg_per_row the host let through
    if (t == 0) {
      a.header->magic = 0;
      a.header->num_items = 0;
    }
    return;
  }

  // Items: split rows first (indices [0, total_multi), one grid round), then
  // one item per whole row.
  for (int r0 = 0; r0 < a.num_rows; r0 += kPlanBlock) {
    const int r = r0 + t;
    int g = 0;
    int64_t c = 0;
    int32_t len = 0;
    if (r < a.num_rows) {
      len = a.lengths[r];
      g = split_of(len, a.k, chunk, force_split, a.wg_per_row, &c);
    }
    const uint32_t n_multi = (r < a.num_rows && g > 1) ? (uint32_t)g : 0u;
    const uint32_t n_group = n_multi ? 1u : 0u;
    const uint32_t n_single = (r < a.num_rows && g == 1) ? 1u : 0u;
    // three scans packed: multi items in 16 bits would overflow, so run them apart
    uint32_t tot_m, tot_g, tot_s;
    const uint32_t off_m = block_exclusive_add(n_multi, s_scan, &tot_m);
    const uint32_t off_g = block_exclusive_add(n_group, s_scan, &tot_g);
    const uint32_t off_s = block_exclusive_add(n_single, s_scan, &tot_s);
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
        w.pad[0] = w.pad[1] = w.pad[2] = 0;
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
      w.pad[0] = w.pad[1] = w.pad[2] = 0;
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
    h.chunk = (int32_t)(chunk > 0x7FFFFFFF ? 0x7FFFFFFF : chunk);
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
// with h the canonical FP16 of x (FP16 order agrees with key order off -0/NaN).
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

struct __align__(16) Smem {
  uint64_t list[kListCap];      // boundary candidates (key32 << 32 | position)
  uint32_t lhist[kBins];        // this workgroup's histogram (raw index)
  uint32_t rhist[kRadixBins];   // refinement digits; also the merged histogram
  uint32_t scratch[kWaves];
  uint32_t res[4];
  uint32_t cur_out;             // next output position of the row
  uint32_t cur_list;            // next candidate position (LDS list or global buffer)
  uint32_t flag;
  uint32_t range[4];            // candidate key/position range: kmax, ~kmin, imax, ~imin
  uint32_t bcast[4];
};

// Output of one row: slot = table[i / ps] * ps + i % ps (page: TopK-V2,
// selected logical positions translated to physical indexer KV-cache slots).
struct RowOut {
  int32_t* slots;
  int32_t* idx;
  const int32_t* table;
  int32_t ps;
  int32_t shift;
  uint32_t k;
  int32_t* status;

  __device__ __forceinline__ void write(uint32_t pos, int32_t i) const {
    if (pos >= k) {  // counts and classification disagree: never write past the row
      atomicOr(status, TOPK_DEVICE_INTERNAL);
      return;
    }
    int32_t page, off;
    if (shift >= 0) {
      page = table[i >> shift];
      off = i & (ps - 1);
    } else {
      page = table[i / ps];
      off = i % ps;
    }
    slots[pos] = page * ps + off;
    if (idx) idx[pos] = i;
  }
};

// Wave-aggregated output: one LDS atomic per wave reserves positions.
__device__ __forceinline__ void emit_wave(bool take, int32_t i, uint32_t* cursor, const RowOut& o) {
  const uint64_t m = __ballot(take);
  if (m == 0) return;
  const uint32_t leader = first_lane(m);
  uint32_t base = 0;
  if (lane() == leader) base = atomicAdd(cursor, (uint32_t)__popcll(m));
  base = read_lane(base, leader);
  if (take) o.write(base + mbcnt(m), i);
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

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, (uint32_t)__shfl_xor(x, d, 64));
  return x;
}

// Element j = q * 4 + c of a lane's tile sits at this position: lane t loads
// dwordx4 number q at (q * kBlock + t) * 4, so each load instruction of a wave
// reads 1 KB of consecutive scores. Packed register hk[j / 2] holds elements
// j & ~1 (low half) and j | 1 (high half).
__device__ __forceinline__ int32_t tile_pos(int32_t base, int q, int c) {
  return base + (q * kBlock + (int)threadIdx.x) * 4 + c;
}

constexpr int kHk = kEpt / 2;   // packed registers per lane

template <bool VEC>
__device__ __forceinline__ void load_pack(const float* rowp, int32_t base, int32_t end, uint32_t (&hk)[kHk]) {
#pragma unroll
  for (int q = 0; q < kEpt / 4; ++q) {
    const int32_t e = tile_pos(base, q, 0);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (VEC) {
      // Rows are 16-byte aligned and their stride is a multiple of 4, so a
      // vector that starts before `end` lies inside the row.
      if (e < end) x = *reinterpret_cast<const float4*>(rowp + e);
    } else {
      if (e < end) x.x = rowp[e];
      if (e + 1 < end) x.y = rowp[e + 1];
      if (e + 2 < end) x.z = rowp[e + 2];
      if (e + 3 < end) x.w = rowp[e + 3];
    }
    uint32_t p0 = to_half2(x.x, x.y), p1 = to_half2(x.z, x.w);
    if (e + 4 > end) {  // tail vector: positions >= end become NaN
      const int n = end - e;
      p0 = n <= 0 ? kHalfNaN2 : (n == 1 ? (p0 & 0xFFFFu) | (kHalfNaN << 16) : p0);
      p1 = n <= 2 ? kHalfNaN2 : (n == 3 ? (p1 & 0xFFFFu) | (kHalfNaN << 16) : p1);
    }
    hk[2 * q] = p0;
    hk[2 * q + 1] = p1;
  }
}

// Histogram of a packed tile. When one bin takes all 256 scores of a wave's
// dwordx4 (all-equal or one-bin rows), a single atomic adds 256 instead of
// 256 conflicting ones. NaN padding lands in an unscanned bin.
__device__ __forceinline__ void hist_packed(const uint32_t (&hk)[kHk], uint32_t* h) {
#pragma unroll
  for (int q = 0; q < kEpt / 4; ++q) {
    const uint32_t p0 = hk[2 * q], p1 = hk[2 * q + 1];
    const uint32_t r0 = (p0 >> 6) & 0x3FFu, r1 = p0 >> 22, r2 = (p1 >> 6) & 0x3FFu, r3 = p1 >> 22;
    const uint32_t f = (uint32_t)__builtin_amdgcn_readfirstlane((int)r0);
    const bool same = r0 == f && r1 == f && r2 == f && r3 == f;
    if (__ballot(same) == ~0ull) {
      if (lane() == 0) atomicAdd(&h[f], 256u);
    } else {
      atomicAdd(&h[r0], 1u);
      atomicAdd(&h[r1], 1u);
      atomicAdd(&h[r2], 1u);
      atomicAdd(&h[r3], 1u);
    }
  }
}

// Bit j set <=> element j lies in the threshold bin or above it.
__device__ __forceinline__ uint32_t interest_mask(const uint32_t (&hk)[kHk], _Float16 vlo) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kHk; ++i) {
    m |= (uint32_t)(half_lo(hk[i]) >= vlo) << (2 * i);
    m |= (uint32_t)(half_hi(hk[i]) >= vlo) << (2 * i + 1);
  }
  return m;
}

// Per-lane running range of the boundary candidates, all kept as maxima.
struct Range {
  uint32_t kmax = 0, kmin_inv = 0, imax = 0, imin_inv = 0;
};

// The few positions of `mask` are re-read as FP32 and classified: above the
// threshold bin -> written to the output; in it -> counted into the range and
// (when cand_dst is set) appended to the candidate list.
__device__ __forceinline__ void extract(uint32_t mask, int32_t base, const float* rowp, _Float16 vhi,
                                        uint32_t* cur_out, const RowOut& o, uint32_t* cur_cand,
                                        uint64_t* cand_dst, uint32_t cand_limit, Range& rg) {
  while (mask) {
    const int j = __builtin_ctz(mask);
    mask &= mask - 1u;
    const int32_t e = tile_pos(base, j >> 2, j & 3);
    const float x = rowp[e];
    if (half_lo(to_half2(x, x)) >= vhi) {
      o.write(atomicAdd(cur_out, 1u), e);
    } else {
      const uint32_t kk = key32_of(x);
      rg.kmax = max(rg.kmax, kk);
      rg.kmin_inv = max(rg.kmin_inv, ~kk);
      rg.imax = max(rg.imax, (uint32_t)e);
      rg.imin_inv = max(rg.imin_inv, ~(uint32_t)e);
      if (cand_dst) {
        const uint32_t c = atomicAdd(cur_cand, 1u);
        if (c < cand_limit) cand_dst[c] = ((uint64_t)kk << 32) | (uint32_t)e;
        else atomicOr(o.status, TOPK_DEVICE_INTERNAL);
      }
    }
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
  uint32_t h[PB];
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const uint32_t b = (uint32_t)(kBins - 1 - (t * PB + j));
    h[j] = (b >= kFirstBin && b <= kLastBin) ? hist[raw_of_bin(b)] : 0u;
    s += h[j];
  }
  uint32_t cum = block_exclusive_add(s, scratch);
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const uint32_t b = (uint32_t)(kBins - 1 - (t * PB + j));
    if (cum < need && need <= cum + h[j]) {
      result[0] = b;
      result[1] = cum;
      result[2] = h[j];
    }
    cum += h[j];
  }
  __syncthreads();
}

// --- candidate sources for the exact refinement -----------------------------
// each(f) calls f(valid, key32, position) for every element slot; the trip
// count is uniform across the workgroup so wave-level ballots stay convergent.

// A packed (key32 << 32 | position) list in LDS or global memory.
struct ListSrc {
  const uint64_t* p;
  uint32_t n;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (uint32_t i0 = 0; i0 < n; i0 += kBlock) {
      const uint32_t i = i0 + threadIdx.x;
      const bool valid = i < n;
      const uint64_t e = valid ? p[i] : 0ull;
      f(valid, (uint32_t)(e >> 32), (int32_t)(uint32_t)e);
    }
  }
};

// Threshold-bin scores of [begin, end), re-read from the row.
template <bool VEC>
struct StreamSrc {
  const float* rowp;
  int32_t begin, end;
  Cut cut;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (int32_t base = begin; base < end; base += 2 * kBlock * 4) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
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
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int32_t e = base + (u * kBlock + (int)threadIdx.x) * 4 + c;
          const _Float16 h = half_lo(to_half2(x[u * 4 + c], 0.f));
          f(e < end && h >= cut.vlo && !(h >= cut.vhi), key32_of(x[u * 4 + c]), e);
        }
    }
  }
};

// Compressed composite key of a boundary candidate: the FP32 key offset from
// the smallest candidate key, then the position reversed so that lower
// positions rank higher. Distinct for distinct positions, so the top `need`
// keys are unique.
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
};

__device__ __forceinline__ uint32_t bit_width(uint32_t x) { return x ? 32u - (uint32_t)__clz(x) : 0u; }

// From the candidate range (kmax, ~kmin, imax, ~imin).
__device__ __forceinline__ Refine make_refine(const uint32_t* range, uint32_t need, uint32_t cnt) {
  Refine p;
  const uint32_t kmax = range[0], kmin = ~range[1], imax = range[2], imin = ~range[3];
  p.lo32 = kmin;
  p.idx_hi = imax;
  p.b2 = bit_width(imax - imin);
  p.nb = bit_width(kmax - kmin) + p.b2;
  p.need = need;
  p.cnt = cnt;
  return p;
}

// Exact selection of the `need` best boundary candidates (FP32 value
// descending, position ascending): MSB-first radix over kRadixBits-bit digits
// of the composite key. Each pass histograms the digit of the candidates that
// match the prefix fixed so far, finds the digit holding the need-th, emits
// the candidates with a larger digit and keeps the equal ones; survivors are
// compacted into LDS as soon as they fit. Outputs go to sh.cur_out onwards.
// SRC_IN_LDS: the source is sh.list itself (no compaction into it).
template <bool SRC_IN_LDS, class Src>
__device__ __forceinline__ void refine(const Src& src, const Refine& p, Smem& sh, const RowOut& o) {
  const int t = threadIdx.x;
  if (p.need == p.cnt) {
    src.each([&](bool valid, uint32_t, int32_t i) { emit_wave(valid, i, &sh.cur_out, o); });
    __syncthreads();
    return;
  }
  uint64_t prefix = 0;
  uint32_t pbits = 0, need = p.need, list_n = 0;
  bool in_list = false;
  for (;;) {
    const uint32_t width = min((uint32_t)kRadixBits, p.nb - pbits);
    const uint32_t shift = p.nb - pbits - width;
    const uint32_t top = shift + width;   // <= 63
    const uint32_t mask = (1u << width) - 1u;
    for (int i = t; i < (int)(mask + 1); i += kBlock) sh.rhist[i] = 0;
    __syncthreads();
    auto hist_fn = [&](bool valid, uint32_t k32, int32_t i) {
      const uint64_t ck = p.key(k32, i);
      hist_add(sh.rhist, valid && (ck >> top) == prefix, (uint32_t)(ck >> shift) & mask);
    };
    if (in_list) ListSrc{sh.list, list_n}.each(hist_fn);
    else src.each(hist_fn);
    __syncthreads();
    if (t == 0) sh.res[0] = kNotFound;
    find_threshold<kRadixBins / kBlock>(sh.rhist, (int)(mask + 1), need, sh.scratch, sh.res);
    if (sh.res[0] == kNotFound) {
      if (t == 0) atomicOr(o.status, TOPK_DEVICE_INTERNAL);
      break;
    }
    const uint32_t d = sh.res[0], above = sh.res[1], cnt = sh.res[2];
    const bool finish = cnt == need - above;
    const bool compact = !SRC_IN_LDS && !in_list && !finish && cnt <= (uint32_t)kListCap;
    if (t == 0) sh.cur_list = 0;
    __syncthreads();
    auto emit_fn = [&](bool valid, uint32_t k32, int32_t i) {
      const uint64_t ck = p.key(k32, i);
      const bool m = valid && (ck >> top) == prefix;
      const uint32_t dig = (uint32_t)(ck >> shift) & mask;
      emit_wave(m && (dig > d || (finish && dig == d)), i, &sh.cur_out, o);
      if (compact) push_wave(m && dig == d, ((uint64_t)k32 << 32) | (uint32_t)i, &sh.cur_list, sh.list);
    };
    if (in_list) ListSrc{sh.list, list_n}.each(emit_fn);
    else src.each(emit_fn);
    __syncthreads();
    if (finish) break;
    need -= above;
    prefix = (prefix << width) | d;
    pbits += width;
    if (compact) {
      in_list = true;
      list_n = cnt;
    }
  }
}

// Out-of-line refinement for the sources outside LDS, so their code does not
// sit in the register-resident path.
template <bool VEC>
__device__ __forceinline__ void refine_stream(const float* rowp, int32_t begin, int32_t end, Cut cut,
                                                        const Refine p, Smem& sh, const RowOut o) {
  refine<false>(StreamSrc<VEC>{rowp, begin, end, cut}, p, sh, o);
}

__device__ __forceinline__ void refine_global(const uint64_t* list, uint32_t n, const Refine p, Smem& sh,
                                                        const RowOut o) {
  refine<false>(ListSrc{list, n}, p, sh, o);
}

// A row the workgroup owns alone: register path when the row fits one tile,
// streaming path otherwise.
template <bool VEC>
__device__ __forceinline__ void owned_row(const SelectArgs& a, int32_t len, const float* rowp, const RowOut& o,
                                          bool resident, uint32_t (&hk)[kHk], Smem& sh) {
  if (threadIdx.x == 0) sh.res[0] = kNotFound;
  find_threshold_raw(sh.lhist, (uint32_t)a.k, sh.scratch, sh.res);
  if (sh.res[0] == kNotFound) {  // fewer valid scores than k: NaN inputs
    if (threadIdx.x == 0) atomicOr(a.status, TOPK_DEVICE_INTERNAL);
    return;
  }
  const uint32_t bstar = sh.res[0], n_above = sh.res[1], cnt = sh.res[2];
  const Cut cut = cut_of_bin(bstar);
  const bool use_list = cnt <= (uint32_t)kListCap;
  if (threadIdx.x == 0) {
    sh.cur_out = 0;
    sh.cur_list = 0;
    sh.range[0] = sh.range[1] = sh.range[2] = sh.range[3] = 0;
  }
  __syncthreads();
  Range rg;
  uint64_t* dst = use_list ? sh.list : nullptr;
  if (resident) {
    extract(interest_mask(hk, cut.vlo), 0, rowp, cut.vhi, &sh.cur_out, o, &sh.cur_list, dst, kListCap, rg);
  } else {
    for (int32_t base = 0; base < len; base += kTile) {
      load_pack<VEC>(rowp, base, len, hk);
      extract(interest_mask(hk, cut.vlo), base, rowp, cut.vhi, &sh.cur_out, o, &sh.cur_list, dst, kListCap, rg);
    }
  }
  merge_range(rg, sh);
  __syncthreads();
  const Refine p = make_refine(sh.range, (uint32_t)a.k - n_above, cnt);
  if (use_list) refine<true>(ListSrc{sh.list, cnt}, p, sh, o);
  else refine_stream<VEC>(rowp, 0, len, cut, p, sh, o);
}

// A row shared by w.gsize workgroups; this one holds chunk [w.begin, end).
template <bool VEC>
__device__ __forceinline__ void split_row(const SelectArgs& a, const WorkItem& w, int32_t len, const float* rowp,
                                          const RowOut& o, bool resident, uint32_t (&hk)[kHk], Smem& sh) {
  const int t = threadIdx.x;
  const int32_t begin = w.begin, end = min(w.end, len);
  const uint32_t G = (uint32_t)w.gsize;
  const uint32_t k = (uint32_t)a.k;
  GroupState* g = a.groups + w.group;

  // Only bins at or above this chunk's own k-th bin can hold the row's k-th.
  uint32_t bloc = 0;
  if ((uint32_t)(end - begin) >= k) {
    if (t == 0) sh.res[0] = 0;
    find_threshold_raw(sh.lhist, k, sh.scratch, sh.res);
    bloc = sh.res[0];
  }
  for (int r = t; r < kBins; r += kBlock) {
    const uint32_t h = sh.lhist[r];
    const uint32_t b = bin_of_raw((uint32_t)r);
    if (h && b >= bloc && b >= kFirstBin && b <= kLastBin)
      __hip_atomic_fetch_add(&g->hist[r], h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (t == 0) {
    __hip_atomic_fetch_add(&g->arrive, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0, ok = 1;
    while (__hip_atomic_load(&g->arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < G) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > a.spin_limit) {
        ok = 0;
        break;
      }
    }
    if (!ok) atomicOr(a.status, TOPK_DEVICE_SPIN_TIMEOUT);
    sh.flag = ok;
  }
  __syncthreads();
  if (!sh.flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int r = t; r < kBins; r += kBlock)
    sh.rhist[r] = __hip_atomic_load(&g->hist[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // Bins at or above the largest chunk threshold are complete, and the row's
  // threshold bin lies there, so the scan from the top is exact.
  if (t == 0) sh.res[0] = kNotFound;
  find_threshold_raw(sh.rhist, k, sh.scratch, sh.res);
  // Not found only with NaN inputs; the workgroup then skips its emission but
  // still takes part in the arrival count so the row's state is reset.
  const bool found = sh.res[0] != kNotFound;
  if (!found && t == 0) atomicOr(a.status, TOPK_DEVICE_INTERNAL);
  const uint32_t bstar = found ? sh.res[0] : kLastBin;
  const uint32_t n_above = found ? sh.res[1] : 0u, cnt = found ? sh.res[2] : 0u;
  const Cut cut = cut_of_bin(bstar);
  uint32_t la = 0;
  for (int r = t; r < kBins; r += kBlock) {
    const uint32_t b = bin_of_raw((uint32_t)r);
    la += (found && b > bstar && b <= kLastBin) ? sh.lhist[r] : 0u;
  }
  uint32_t local_above;
  block_exclusive_add(la, sh.scratch, &local_above);
  const uint32_t local_cnt = found ? sh.lhist[raw_of_bin(bstar)] : 0u;
  const bool keep = found && (int64_t)cnt <= a.cand_cap;
  uint32_t base_out = 0, base_cand = 0;
  if (t == 0) {
    if (local_above) base_out = __hip_atomic_fetch_add(&g->emit, local_above, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (keep && local_cnt) base_cand = __hip_atomic_fetch_add(&g->cand, local_cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the interest mask overlaps the two atomics' round trip
  const uint32_t mask0 = (resident && found) ? interest_mask(hk, cut.vlo) : 0u;
  if (t == 0) {
    sh.cur_out = base_out;
    sh.cur_list = base_cand;
    sh.range[0] = sh.range[1] = sh.range[2] = sh.range[3] = 0;
  }
  __syncthreads();
  uint64_t* slab = a.cand + (int64_t)w.group * a.cand_cap;
  uint64_t* dst = keep ? slab : nullptr;
  Range rg;
  if (resident) {
    extract(mask0, begin, rowp, cut.vhi, &sh.cur_out, o, &sh.cur_list, dst, (uint32_t)a.cand_cap, rg);
  } else if (found) {
    for (int32_t base = begin; base < end; base += kTile) {
      load_pack<VEC>(rowp, base, end, hk);
      extract(interest_mask(hk, cut.vlo), base, rowp, cut.vhi, &sh.cur_out, o, &sh.cur_list, dst,
              (uint32_t)a.cand_cap, rg);
    }
  }
  merge_range(rg, sh);
  __syncthreads();
  if (t == 0) {
    if (local_cnt) {
      __hip_atomic_fetch_max(&g->range[0], sh.range[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(&g->range[1], sh.range[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(&g->range[2], sh.range[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(&g->range[3], sh.range[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (t == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&g->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = prev == G - 1;
  }
  __syncthreads();
  if (!sh.flag) return;
  // Last workgroup of the row: resolve the threshold bin.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (t < 4) sh.range[t] = __hip_atomic_load(&g->range[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t == 0) sh.cur_out = n_above;
  __syncthreads();
  const Refine p = make_refine(sh.range, k - n_above, cnt);
  if (!found) {
  } else if (keep) {
    refine_global(slab, cnt, p, sh, o);
  } else {
    refine_stream<VEC>(rowp, 0, len, cut, p, sh, o);
  }
  for (int r = t; r < kBins; r += kBlock) __hip_atomic_store(&g->hist[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t < 4) __hip_atomic_store(&g->range[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t == 0) {
    __hip_atomic_store(&g->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&g->emit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&g->cand, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&g->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool VEC>
__device__ __forceinline__ void process_item(const SelectArgs& a, const WorkItem& w, Smem& sh) {
  const int t = threadIdx.x;
  const int row = w.row;
  const int32_t len = a.lengths[row];
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
  o.status = a.status;
  if (len <= a.k) {  // every valid position is selected; pad with -1
    if (w.begin == 0) {
      for (int j = t; j < a.k; j += kBlock) {
        if (j < len) {
          o.write((uint32_t)j, j);
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
  const bool resident = end - begin <= kTile;
  uint32_t hk[kHk];
  for (int i = t; i < kBins; i += kBlock) sh.lhist[i] = 0;
  __syncthreads();
  if (resident) {
    load_pack<VEC>(rowp, begin, end, hk);
    hist_packed(hk, sh.lhist);
  } else {
    for (int32_t base = begin; base < end; base += kTile) {
      load_pack<VEC>(rowp, base, end, hk);
      hist_packed(hk, sh.lhist);
    }
  }
  __syncthreads();
  if (w.group < 0) owned_row<VEC>(a, len, rowp, o, resident, hk, sh);
  else split_row<VEC>(a, w, len, rowp, o, resident, hk, sh);
}

template <bool VEC>
__global__ void __launch_bounds__(kBlock, 4) topk_select_kernel(SelectArgs a) {
  __shared__ Smem sh;
  const PlanHeader h = *a.plan;
  if (h.magic != kPlanMagic || h.k != a.k || h.grid != (int)gridDim.x || h.num_rows > a.num_rows) {
    if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(a.status, TOPK_DEVICE_PLAN_MISMATCH);
    return;
  }
  for (int it = blockIdx.x; it < h.num_items; it += gridDim.x) {
    const WorkItem w = a.items[it];
    process_item<VEC>(a, w, sh);
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

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI in topk_api.hip).
// ---------------------------------------------------------------------------
hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_plan_kernel, dim3(1), dim3(kPlanBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, int grid, bool vec, hipStream_t s) {
  if (vec) hipLaunchKernelGGL(topk_select_kernel<true>, dim3(grid), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL(topk_select_kernel<false>, dim3(grid), dim3(kBlock), 0, s, a);
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

hipError_t select_occupancy(int* per_cu) {
  int a = 0, b = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, (const void*)topk_select_kernel<true>, kBlock, 0);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)topk_select_kernel<false>, kBlock, 0);
  if (e != hipSuccess) return e;
  *per_cu = a < b ? a : b;
  return hipSuccess;
}

}  // namespace satopk
