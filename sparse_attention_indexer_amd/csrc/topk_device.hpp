// topk_device.hpp -- gfx950 device helpers of the indexer top-k library:
// ordered keys, wave64 primitives, block scans and LDS histograms.
#pragma once

#include <hip/hip_runtime.h>

#include "topk_layout.hpp"

namespace satopk {

// ---------------------------------------------------------------------------
// Ordered keys. The lmsys.org TopK-V2 section (Figure 3 caption) maps each
// score to an unsigned key ordered like the score: flip all bits of a
// negative value, set the sign bit of a non-negative one, which turns
// sign-magnitude order into unsigned order. -0.0 is first replaced by +0.0 (a
// test on the bit pattern, so no denormal is flushed) because the two scores
// are equal and must share a key. This FP32 key drives the exact boundary
// refinement; the FP16 histogram key lives with the selection kernel.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t canon_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return b == 0x80000000u ? 0u : b;
}

__device__ __forceinline__ uint32_t key32_of(float x) {
  const uint32_t b = canon_bits(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------
// wave64 primitives
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lane() { return __lane_id(); }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t first_lane(uint64_t m) {
  return (uint32_t)__builtin_ctzll(m);
}

// Zero in a vector register, produced by an instruction the compiler cannot
// see through: an address offset by it is divergent to the compiler.
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// A value every lane holds equally (an LDS broadcast), moved to a scalar
// register so that it costs no VGPR and branches on it stay uniform.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

__device__ __forceinline__ uint32_t read_lane(uint32_t v, uint32_t l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)l);
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, d, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), d, 64);
    x += ((uint64_t)hi << 32) | lo;
  }
  return x;
}

// Wave64 inclusive prefix sum with DPP lane moves: row_shr 1/2/4/8 scan each
// 16-lane row, row_bcast 15/31 carry row totals forward (rows 1,3 then 2,3).
// A few VALU operations instead of six LDS cross-lane round trips.
#define SATOPK_DPP(x, ctrl, rmask) ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x), (ctrl), (rmask), 0xf, false))
__device__ __forceinline__ uint32_t wave_inclusive_add(uint32_t x) {
  x += SATOPK_DPP(x, 0x111, 0xf);  // row_shr:1
  x += SATOPK_DPP(x, 0x112, 0xf);  // row_shr:2
  x += SATOPK_DPP(x, 0x114, 0xf);  // row_shr:4
  x += SATOPK_DPP(x, 0x118, 0xf);  // row_shr:8
  x += SATOPK_DPP(x, 0x142, 0xa);  // row_bcast:15
  x += SATOPK_DPP(x, 0x143, 0xc);  // row_bcast:31
  return x;
}

// Sum over the wave (every lane receives it).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_add(x), 63);
}

// Maximum over the wave (every lane receives it).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, SATOPK_DPP(x, 0x111, 0xf));
  x = max(x, SATOPK_DPP(x, 0x112, 0xf));
  x = max(x, SATOPK_DPP(x, 0x114, 0xf));
  x = max(x, SATOPK_DPP(x, 0x118, 0xf));
  x = max(x, SATOPK_DPP(x, 0x142, 0xa));
  x = max(x, SATOPK_DPP(x, 0x143, 0xc));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Exclusive prefix sum over a workgroup of NW waves, in thread order.
// `scratch` holds NW words of LDS. Every thread must call it.
template <int NW = kWaves>
__device__ __forceinline__ uint32_t block_exclusive_add(uint32_t x, uint32_t* scratch,
                                                        uint32_t* total = nullptr) {
  const uint32_t w = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_add(x);
  if (lane() == 63) scratch[w] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = scratch[i];
    pre += ((uint32_t)i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  if (total) *total = tot;
  return pre + inc - x;
}

// LDS histogram increment, aggregated per wave: when every active lane hits
// the same bin (all-equal or one-bin rows) one atomic adds the lane count
// instead of 64 conflicting atomics. Must be called by the whole wave.
__device__ __forceinline__ void hist_add(uint32_t* h, bool m, uint32_t bin) {
  const uint64_t act = __ballot(m);
  if (act == 0) return;
  const uint32_t leader = first_lane(act);
  const uint32_t b0 = read_lane(bin, leader);
  const uint64_t same = __ballot(m && bin == b0);
  if (same == act) {
    if (lane() == leader) atomicAdd(&h[b0], (uint32_t)__popcll(act));
  } else if (m) {
    atomicAdd(&h[bin], 1u);
  }
}

// Scan `nb` bins from the top and find the bin holding the need-th largest
// element: above(b) < need <= above(b) + h[b]. Writes (b, above(b), h[b]) to
// result[0..2]. PB bins per thread; nb <= PB * kBlock; 1 <= need <= sum(h).
// Bin b lives at hist[b + (b >> PAD)] when PAD > 0: one pad word per 2^PAD
// bins keeps the lanes' contiguous PB-bin reads on distinct LDS banks.
template <int PB, int PAD = 0>
__device__ __forceinline__ uint32_t bin_addr(int b) { return PAD ? (uint32_t)(b + (b >> PAD)) : (uint32_t)b; }

template <int PB, int PAD = 0>
__device__ __forceinline__ void find_threshold(const uint32_t* hist, int nb, uint32_t need,
                                               uint32_t* scratch, uint32_t* result) {
  const int t = threadIdx.x;
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const int b = nb - 1 - (t * PB + j);
    s += b >= 0 ? hist[bin_addr<PB, PAD>(b)] : 0u;
  }
  const uint32_t cum = block_exclusive_add(s, scratch);
  // The wave holding the thread whose bins straddle `need` resolves them in
  // parallel: lane l < PB takes that thread's l-th bin, and a 16-lane DPP
  // prefix sum replaces a serial rescan of dependent LDS reads.
  static_assert(PB <= 16, "one DPP row holds the straddling thread's bins");
  const uint64_t strad = __ballot(cum < need && need <= cum + s);
  if (strad) {
    const uint32_t sl = first_lane(strad);
    const uint32_t c0 = read_lane(cum, sl);
    const int ts = (t & ~63) + (int)sl;
    const int l = (int)lane();
    const int b = nb - 1 - (ts * PB + l);
    const uint32_t h = (l < PB && b >= 0) ? hist[bin_addr<PB, PAD>(b)] : 0u;
    uint32_t inc = h;
    inc += SATOPK_DPP(inc, 0x111, 0xf);  // row_shr:1
    inc += SATOPK_DPP(inc, 0x112, 0xf);  // row_shr:2
    inc += SATOPK_DPP(inc, 0x114, 0xf);  // row_shr:4
    inc += SATOPK_DPP(inc, 0x118, 0xf);  // row_shr:8
    if (l < PB && c0 + inc - h < need && need <= c0 + inc) {
      result[0] = (uint32_t)b;
      result[1] = c0 + inc - h;
      result[2] = h;
    }
  }
  __syncthreads();
}

}  // namespace satopk
