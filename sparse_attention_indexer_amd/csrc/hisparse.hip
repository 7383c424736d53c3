// hisparse.hip -- the HiSparse top-k resolver for gfx950 (vllm.ai page "GLM
// 5.3 Optimizations, Part 1: Hybrid HiSparse Offloading in vLLM", section
// "How it works"; the rule the library implements is in hisparse.h).
//
// One 512-lane workgroup per request and decode step:
//  1. every selected position is classified at once (one lane each):
//     resident pages give their row, hot hits refresh their stamp, misses are
//     appended to an LDS list as (position, output index) keys;
//  2. the misses are sorted by position and the hot slots by (stamp, slot),
//     slots used in this step sorting last (bitonic sorts in LDS);
//  3. miss i takes slot i: the old tag is unmapped, the new one mapped and
//     stamped, and the output row written;
//  4. the missed rows are copied from pinned host memory (read through its
//     device mapping, 16 bytes per lane and load) into their hot KV rows.
#include <hip/hip_runtime.h>

#include "hisparse.h"

namespace satopk {
namespace {

constexpr int kHsBlock = 512;
constexpr int kHsMaxK = 2048;
constexpr int kHsMaxHot = 4096;

struct HsArgs {
  uint32_t step;
  int32_t k, hot, page_size, max_ctx, row_bytes;
  const int32_t* sel;
  int64_t sel_stride;
  const int32_t* table;
  int64_t bt_stride;
  const int32_t* host_table;
  int64_t host_bt_stride;
  const int64_t* hot_rows;
  int32_t* tag;
  uint32_t* stamp;
  int32_t* map;
  uint8_t* kv;
  int64_t kv_rows;
  const uint8_t* host;   // device mapping of the pinned host pool
  int64_t host_rows;
  int64_t* rows_out;
  int32_t* status;
};

// Ascending bitonic sort of n (a power of two) keys in LDS by the whole
// workgroup; pairs (lo, lo + stride) with lo's `stride` bit clear.
__device__ void bitonic_sort(uint64_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += kHsBlock) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 2;
  while (p < n) p <<= 1;
  return p;
}

__global__ void __launch_bounds__(kHsBlock) hisparse_kernel(HsArgs a) {
  __shared__ uint64_t miss[kHsMaxK];
  __shared__ uint64_t vict[kHsMaxHot];
  __shared__ uint32_t n_miss;
  __shared__ int32_t flags;
  const int t = threadIdx.x;
  const int r = blockIdx.x;
  const int32_t* sel = a.sel + (int64_t)r * a.sel_stride;
  const int32_t* table = a.table + (int64_t)r * a.bt_stride;
  const int32_t* host_table = a.host_table + (int64_t)r * a.host_bt_stride;
  const int64_t* hot_rows = a.hot_rows + (int64_t)r * a.hot;
  int32_t* tag = a.tag + (int64_t)r * a.hot;
  uint32_t* stamp = a.stamp + (int64_t)r * a.hot;
  int32_t* map = a.map + (int64_t)r * a.max_ctx;
  int64_t* out = a.rows_out + (int64_t)r * a.k;
  if (t == 0) {
    n_miss = 0;
    flags = 0;
  }
  __syncthreads();
  // 1. classify
  for (int j = t; j < a.k; j += kHsBlock) {
    const int32_t p = sel[j];
    int64_t row = -1;
    if (p >= a.max_ctx) {
      atomicOr(&flags, HISPARSE_DEVICE_BAD_INDEX);
    } else if (p >= 0) {
      const int32_t page = table[p / a.page_size];
      if (page >= 0) {
        row = (int64_t)page * a.page_size + p % a.page_size;
      } else {
        const int32_t s = map[p];
        if (s >= a.hot) {
          atomicOr(&flags, HISPARSE_DEVICE_BAD_INDEX);   // a state array holds a slot past the hot buffer
        } else if (s >= 0) {
          stamp[s] = a.step;
          row = hot_rows[s];
        } else {
          miss[atomicAdd(&n_miss, 1u)] = ((uint64_t)(uint32_t)p << 32) | (uint32_t)j;
        }
      }
    }
    out[j] = row;   // misses are overwritten below
  }
  __syncthreads();
  const int m = (int)n_miss;
  if (m > 0) {
    // 2. misses by position; slots by (stamp, slot), this step's last
    const int mp = pow2_at_least(m), hp = pow2_at_least(a.hot);
    for (int i = m + t; i < mp; i += kHsBlock) miss[i] = ~0ull;
    for (int s = t; s < hp; s += kHsBlock) {
      uint64_t key = ~0ull;
      if (s < a.hot) {
        const uint32_t st = stamp[s];
        if (st != a.step) key = ((uint64_t)st << 32) | (uint32_t)s;
      }
      vict[s] = key;
    }
    __syncthreads();
    bitonic_sort(miss, mp);
    bitonic_sort(vict, hp);
    // 3. assign
    for (int i = t; i < m; i += kHsBlock) {
      const int32_t p = (int32_t)(miss[i] >> 32);
      const int j = (int)(uint32_t)miss[i];
      const uint64_t v = i < hp ? vict[i] : ~0ull;   // (fewer slots than misses)
      int64_t row = -1;
      if (v == ~0ull) {
        atomicOr(&flags, HISPARSE_DEVICE_HOT_FULL);
      } else {
        const int s = (int)(uint32_t)v;
        const int64_t kv_row = hot_rows[s];
        const int64_t host_row = (int64_t)host_table[p / a.page_size] * a.page_size + p % a.page_size;
        if (kv_row < 0 || kv_row >= a.kv_rows || host_row < 0 || host_row >= a.host_rows) {
          atomicOr(&flags, HISPARSE_DEVICE_BAD_INDEX);
          vict[i] = ~0ull;   // (no copy below; i < hp here)
        } else {
          const int32_t old = tag[s];
          if (old >= 0 && old < a.max_ctx) map[old] = -1;
          tag[s] = p;
          map[p] = s;
          stamp[s] = a.step;
          row = kv_row;
          miss[i] = ((uint64_t)(uint64_t)host_row << 32) | (uint32_t)s;   // host row and slot for the copy
        }
      }
      out[j] = row;
    }
    __syncthreads();
    // 4. copy the missed rows from host memory, 16 bytes per lane and load
    // (batching eight loads per lane before their stores timed the same: the
    // copy is bound by the host link, about 27 GB/s of these reads)
    const int chunks = a.row_bytes / 16;
    const int64_t total = (int64_t)m * chunks;
    for (int64_t u = t; u < total; u += kHsBlock) {
      const int i = (int)(u / chunks), c = (int)(u % chunks);
      if (i >= hp || vict[i] == ~0ull) continue;
      const int s = (int)(uint32_t)miss[i];
      const int64_t host_row = (int64_t)(miss[i] >> 32);
      const uint4 x = *reinterpret_cast<const uint4*>(a.host + host_row * a.row_bytes + c * 16);
      *reinterpret_cast<uint4*>(a.kv + hot_rows[s] * a.row_bytes + c * 16) = x;
    }
  }
  __syncthreads();
  if (t == 0 && flags && a.status) atomicOr(a.status, flags);
}

}  // namespace
}  // namespace satopk

using namespace satopk;

extern "C" {

topk_status hisparse_resolve(const hisparse_config* cfg, uint32_t step, int32_t requests, const int32_t* sel,
                             int64_t sel_stride, const int32_t* block_table, int64_t bt_stride,
                             const int32_t* host_table, int64_t host_bt_stride, const int64_t* hot_rows,
                             int32_t* tag, uint32_t* stamp, int32_t* map, uint8_t* kv, int64_t kv_rows,
                             const uint8_t* host_pool, int64_t host_rows, int64_t* rows_out, int32_t* status,
                             void* stream) {
  if (!cfg || cfg->k < 1 || cfg->k > kHsMaxK || cfg->hot < 1 || cfg->hot > kHsMaxHot || cfg->page_size < 1 ||
      cfg->max_ctx < 1 || cfg->row_bytes < 16 || cfg->row_bytes % 16 != 0)
    return TOPK_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (cfg->reserved[i] != 0) return TOPK_ERR_INVALID_ARG;
  const int64_t pages = ((int64_t)cfg->max_ctx + cfg->page_size - 1) / cfg->page_size;
  if (step == 0 || requests < 0 || sel_stride < cfg->k || kv_rows < 1 || host_rows < 1 || host_rows > 0x7FFFFFFF)
    return TOPK_ERR_INVALID_ARG;
  if (requests > 1 && (bt_stride < pages || host_bt_stride < pages)) return TOPK_ERR_INVALID_ARG;
  if (requests == 0) return TOPK_OK;
  if (!sel || !block_table || !host_table || !hot_rows || !tag || !stamp || !map || !kv || !host_pool || !rows_out)
    return TOPK_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(kv) & 15u) || (reinterpret_cast<uintptr_t>(host_pool) & 15u))
    return TOPK_ERR_INVALID_ARG;
  // The host pool must be host memory that the device can read; the kernel
  // uses the device's mapping of it.
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_pool) != hipSuccess) {
    (void)hipGetLastError();   // (clear the lookup's error: the pointer is unknown to HIP)
    return TOPK_ERR_INVALID_ARG;
  }
  if (attr.type != hipMemoryTypeHost || !attr.devicePointer) return TOPK_ERR_INVALID_ARG;
  HsArgs a;
  a.step = step;
  a.k = cfg->k;
  a.hot = cfg->hot;
  a.page_size = cfg->page_size;
  a.max_ctx = cfg->max_ctx;
  a.row_bytes = cfg->row_bytes;
  a.sel = sel;
  a.sel_stride = sel_stride;
  a.table = block_table;
  a.bt_stride = bt_stride;
  a.host_table = host_table;
  a.host_bt_stride = host_bt_stride;
  a.hot_rows = hot_rows;
  a.tag = tag;
  a.stamp = stamp;
  a.map = map;
  a.kv = kv;
  a.kv_rows = kv_rows;
  a.host = static_cast<const uint8_t*>(attr.devicePointer);
  a.host_rows = host_rows;
  a.rows_out = rows_out;
  a.status = status;
  hipLaunchKernelGGL(hisparse_kernel, dim3((unsigned)requests), dim3(kHsBlock), 0, static_cast<hipStream_t>(stream),
                     a);
  return hipGetLastError() == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

}  // extern "C"
