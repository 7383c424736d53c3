// logits.hip -- the indexer's score producer for gfx950: MQA logits of a few
// query tokens against the paged FP8 key cache on the MFMA matrix cores,
// written as the FP32 score rows the top-k selection reads (lmsys page
// "Serving GLM5.2 NVFP4 Agentic Workload with SGLang", sections "Kernel
// Optimization / TopK-V2" and "What's Next"; the score formula the library
// implements is in indexer_logits.h).
//
// The contraction: for every key s, C[t*H + h][s] = q_codes[t][h] . k_codes[s]
// over D = 128, an (T*H) x 128 by 128 x (keys) product in FP8 E4M3 with FP32
// accumulation (v_mfma_f32_32x32x64_f8f6f4: a 32x64 by 64x32 block per
// instruction, two instructions per 128-deep dot). Keys are the N dimension,
// 32 per wave step; each wave loads its 32 keys once (four 16-byte loads per
// lane, straight from the key's cache row) and multiplies them by every
// query row, which the workgroup keeps in LDS. The epilogue folds each 32x32
// block: a lane holds one key and 16 of the 32 heads of the block, so
// ReLU, the head-gate weights and the head sum stay in the lane, and one
// cross-half exchange adds the other 16 heads. The query rows sit in LDS
// with their eight 16-byte chunks XOR-swizzled by the row's low three bits:
// the 32 lanes of a half-wave read one chunk of 32 consecutive rows, 128
// bytes apart, which would otherwise all fall in the same banks.
#include <hip/hip_runtime.h>

#include "indexer_logits.h"

namespace satopk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kDim = 128;
constexpr int kLgBlock = 512;              // 8 waves share one copy of the queries in LDS
constexpr int kLgWaves = kLgBlock / 64;
constexpr int kKeysPerStep = 32;           // N of one MFMA block
constexpr int kMaxQRows = INDEXER_LOGITS_MAX_QROWS;   // tokens x heads held in LDS
static_assert(kMaxQRows * kDim <= 64 * 1024, "query codes fit 64 KB of LDS (two workgroups per CU)");

struct LogitsArgs {
  const uint8_t* q;        // [T][H][128]
  const float* w;          // [T][H]
  int32_t tokens;
  int32_t heads;
  const uint8_t* k;        // [slots][128]
  const float* k_scale;    // [slots]
  const int32_t* table;    // the request's block-table row
  int32_t page_size;
  int32_t page_shift;      // log2(page_size) when a power of two, else -1
  int64_t num_slots;
  const int32_t* lengths;  // [T]
  int32_t max_len;         // max over lengths (host-supplied bound)
  float* out;              // [T][out_stride]
  int64_t out_stride;
  int32_t* status;
};

// The 32 keys of one step: this lane's key row halves (B operands) and scale.
struct KeyStep {
  v8i b0, b1;
  float scale;
  bool ok;    // a valid key whose slot lies in the cache
  bool bad;   // a valid key whose table entry points outside the cache
};

__device__ __forceinline__ KeyStep load_keys(const LogitsArgs& a, int32_t s, int half) {
  KeyStep k;
  k.b0 = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  k.b1 = k.b0;
  k.scale = 0.f;
  k.ok = false;
  k.bad = false;
  if (s < a.max_len) {
    const int32_t page = a.table[a.page_shift >= 0 ? s >> a.page_shift : s / a.page_size];
    const int64_t slot =
        (int64_t)page * a.page_size + (a.page_shift >= 0 ? s & (a.page_size - 1) : s % a.page_size);
    if (page < 0 || slot >= a.num_slots) {
      k.bad = true;
    } else {
      // dims [32 half, +32) and [64 + 32 half, +32) of the key's row
      const uint4* kr = reinterpret_cast<const uint4*>(a.k + slot * kDim + half * 32);
      const uint4 x0 = kr[0], x1 = kr[1], x2 = kr[4], x3 = kr[5];
      k.b0 = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      k.b1 = v8i{(int)x2.x, (int)x2.y, (int)x2.z, (int)x2.w, (int)x3.x, (int)x3.y, (int)x3.z, (int)x3.w};
      k.scale = a.k_scale[slot];
      k.ok = true;
    }
  }
  return k;
}

// HB = heads / 32 head blocks per token, unrolled so that the blocks' matrix
// instructions are independent of one another's epilogues. Each wave works
// through its steps with the next step's key loads in flight.
template <int HB>
__global__ void __launch_bounds__(kLgBlock, 2) mqa_logits_kernel(LogitsArgs a) {
  __shared__ __align__(16) uint8_t qs[kMaxQRows * kDim];
  __shared__ __align__(16) float ws[kMaxQRows];
  __shared__ int32_t lens[64];
  constexpr int H = 32 * HB;
  const int t = threadIdx.x;
  const int rows = a.tokens * H;
  // Stage the query codes (chunk c of row r at chunk c ^ (r & 7)), the gate
  // weights and the lengths.
  for (int i = t; i < rows * kDim / 16; i += kLgBlock)
    reinterpret_cast<uint4*>(qs)[(i & ~7) | ((i & 7) ^ ((i >> 3) & 7))] = reinterpret_cast<const uint4*>(a.q)[i];
  for (int i = t; i < rows; i += kLgBlock) ws[i] = a.w[i];
  if (t < a.tokens) lens[t] = min(a.lengths[t], a.max_len);
  __syncthreads();

  const int l = t & 63;
  const int n = l & 31;          // this lane's key within the step (B column, C column)
  const int half = l >> 5;       // which 32 of each 64-deep block (A/B), which 4-row group (C)
  // Byte offsets of the lane's four A chunks (2 half, +1, +4, +5) in its
  // swizzled query row: every row it reads has row & 7 == n & 7.
  const int sw = n & 7;
  const int c0 = ((2 * half) ^ sw) * 16, c1 = ((2 * half + 1) ^ sw) * 16;
  const int c2 = ((2 * half + 4) ^ sw) * 16, c3 = ((2 * half + 5) ^ sw) * 16;
  const int64_t steps = ((int64_t)a.max_len + kKeysPerStep - 1) / kKeysPerStep;
  const int64_t stride = (int64_t)gridDim.x * kLgWaves;
  int64_t step = (int64_t)blockIdx.x * kLgWaves + (t >> 6);
  KeyStep cur = load_keys(a, step < steps ? (int32_t)(step * kKeysPerStep) + n : a.max_len, half);
  for (; step < steps; step += stride) {
    const int64_t next = step + stride;
    const KeyStep nxt = load_keys(a, next < steps ? (int32_t)(next * kKeysPerStep) + n : a.max_len, half);
    const int32_t s = (int32_t)(step * kKeysPerStep) + n;
    if (cur.bad && a.status) atomicOr(a.status, INDEXER_DEVICE_BAD_SLOT);
    for (int tok = 0; tok < a.tokens; ++tok) {
      v16f acc[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        // A: query rows tok*H + 32 hb + (0..31), the same dims as the key operand
        const uint8_t* qr = qs + (size_t)(tok * H + 32 * hb + n) * kDim;
        const uint4 y0 = *reinterpret_cast<const uint4*>(qr + c0), y1 = *reinterpret_cast<const uint4*>(qr + c1);
        const uint4 y2 = *reinterpret_cast<const uint4*>(qr + c2), y3 = *reinterpret_cast<const uint4*>(qr + c3);
        const v8i a0 = {(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
        const v8i a1 = {(int)y2.x, (int)y2.y, (int)y2.z, (int)y2.w, (int)y3.x, (int)y3.y, (int)y3.z, (int)y3.w};
        acc[hb] = v16f{};
        // FP8 E4M3 operands (format code 0 for both), no block scales
        acc[hb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, cur.b0, acc[hb], 0, 0, 0, 0, 0, 0);
        acc[hb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, cur.b1, acc[hb], 0, 0, 0, 0, 0, 0);
      }
      float total = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        // acc[hb][r] is head 32 hb + 8 (r / 4) + 4 half + r % 4 of this lane's key
        const float* wr = ws + tok * H + 32 * hb + 4 * half;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 wv = *reinterpret_cast<const float4*>(wr + 8 * g);
          total += wv.x * fmaxf(acc[hb][4 * g + 0], 0.f);
          total += wv.y * fmaxf(acc[hb][4 * g + 1], 0.f);
          total += wv.z * fmaxf(acc[hb][4 * g + 2], 0.f);
          total += wv.w * fmaxf(acc[hb][4 * g + 3], 0.f);
        }
      }
      // The other 16 heads of each block, same key: after the swap, lane n < 32
      // holds its own total and lane n + 32's.
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(total), __float_as_uint(total), false, false);
      total = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
      if (half == 0 && cur.ok && s < lens[tok]) a.out[(int64_t)tok * a.out_stride + s] = total * cur.scale;
    }
    cur = nxt;
  }
}

}  // namespace
}  // namespace satopk

using namespace satopk;

extern "C" {

topk_status indexer_mqa_logits(const uint8_t* q_codes, const float* w, int32_t tokens, int32_t heads,
                               const uint8_t* k_fp8, const float* k_scale, int64_t num_slots,
                               const int32_t* block_table, int32_t page_size, const int32_t* lengths,
                               int32_t max_len, float* out, int64_t out_stride, int32_t* status, void* stream) {
  if (tokens < 0 || !(heads == 32 || heads == 64 || heads == 128) || page_size < 1 || max_len < 0 ||
      num_slots < 1 || out_stride < max_len)
    return TOPK_ERR_INVALID_ARG;
  if ((int64_t)tokens * heads > kMaxQRows || tokens > 64) return TOPK_ERR_UNSUPPORTED;
  if (tokens == 0 || max_len == 0) return TOPK_OK;
  if (!q_codes || !w || !k_fp8 || !k_scale || !block_table || !lengths || !out) return TOPK_ERR_INVALID_ARG;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (misaligned(q_codes) || misaligned(w) || misaligned(k_fp8)) return TOPK_ERR_INVALID_ARG;
  LogitsArgs a;
  a.q = q_codes;
  a.w = w;
  a.tokens = tokens;
  a.heads = heads;
  a.k = k_fp8;
  a.k_scale = k_scale;
  a.table = block_table;
  a.page_size = page_size;
  a.page_shift = (page_size & (page_size - 1)) == 0 ? __builtin_ctz((unsigned)page_size) : -1;
  a.num_slots = num_slots;
  a.lengths = lengths;
  a.max_len = max_len;
  a.out = out;
  a.out_stride = out_stride;
  a.status = status;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return TOPK_ERR_HIP;
  const int64_t steps = ((int64_t)max_len + kKeysPerStep - 1) / kKeysPerStep;
  int64_t blocks = (steps + kLgWaves - 1) / kLgWaves;
  if (blocks > 2 * (int64_t)cus) blocks = 2 * (int64_t)cus;   // two resident workgroups per CU, persistent
  const dim3 grid((unsigned)blocks), block(kLgBlock);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (heads == 32) hipLaunchKernelGGL(mqa_logits_kernel<1>, grid, block, 0, st, a);
  else if (heads == 64) hipLaunchKernelGGL(mqa_logits_kernel<2>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(mqa_logits_kernel<4>, grid, block, 0, st, a);
  return hipGetLastError() == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

}  // extern "C"
