// prologue.hip -- the fused indexer key prologue for gfx950: LayerNorm,
// rotary embedding, FP8 E4M3 quantization and the paged indexer-cache store
// of each new key token, in one kernel (lmsys page "Serving GLM5.2 NVFP4
// Agentic Workload with SGLang", section "Indexer Prologue Fusion", key
// path; the formulas the library implements are in indexer_prologue.h).
//
// Layout of the work: 16 lanes per token, 8 of the 128 dimensions per lane
// (one 16-byte BF16 load, one 8-byte FP8 store), kTokensPerGroup tokens per
// 16-lane group. The token's reductions (mean, variance, amax) stay inside
// its 16 lanes; rotary pairs (2i, 2i+1) never straddle lanes. The path is
// bound by memory traffic (about 430 bytes per token), so every load is 16
// bytes wide and every store contiguous per token.
#include <hip/hip_runtime.h>

#include "indexer_prologue.h"

namespace satopk {
namespace {

constexpr int kKeyDim = INDEXER_KEY_DIM;
constexpr int kLanesPerToken = 16;
constexpr int kDimsPerLane = kKeyDim / kLanesPerToken;   // 8
constexpr int kPrologueBlock = 256;
constexpr int kGroupsPerBlock = kPrologueBlock / kLanesPerToken;   // 16-lane token groups
constexpr int kTokensPerGroup = 1;   // 2 timed the same, 4 slower (fewer waves in flight)
constexpr int kTokensPerBlock = kGroupsPerBlock * kTokensPerGroup;
static_assert(kDimsPerLane == 8, "one 16-byte BF16 load per lane");

constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxFloor = 5.42101086242752217e-20f;   // 2^-64: 448 / amax stays finite

struct KeyArgs {
  const uint16_t* k_act;
  int64_t k_stride;
  int32_t num_tokens;
  const float* weight;
  const float* bias;
  float eps;
  const float* cos_sin;
  int32_t rope_dim;
  int32_t max_pos;
  const int32_t* positions;
  const int32_t* token_row;
  const int32_t* table;
  int64_t table_stride;
  int32_t page_size;
  uint8_t* cache_fp8;
  float* cache_scale;
  int64_t num_slots;
  int32_t* status;
};

// Sum / max over the 16 lanes of the calling lane's token group.
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, kLanesPerToken);
  return v;
}
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kLanesPerToken));
  return v;
}

// Two FP32 values to E4M3 (fn) codes in bytes `HI ? 2, 3 : 0, 1` of `old`,
// round to nearest even; inputs are clamped to +-448 first so that nothing
// overflows (the conversion itself has no saturating form to rely on).
template <bool HI>
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// One token's work on its 16 lanes, given the loads already made.
__device__ __forceinline__ void key_token(const KeyArgs& a, int sub, int32_t pos, int32_t page, uint4 raw,
                                          const float (&w)[kDimsPerLane], const float (&bb)[kDimsPerLane],
                                          float4 c, float4 s) {
  // BF16 -> FP32: the 16 bits are the top half of the FP32 word.
  const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[kDimsPerLane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(words[i] << 16);
    x[2 * i + 1] = __uint_as_float(words[i] & 0xFFFF0000u);
  }
  // LayerNorm: mean, then the biased variance of the centred values.
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) sum += x[i];
  const float mean = group_sum(sum) * (1.0f / kKeyDim);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) {
    x[i] -= mean;
    sq += x[i] * x[i];
  }
  const float var = group_sum(sq) * (1.0f / kKeyDim);
  const float rstd = 1.0f / sqrtf(var + a.eps);
  float y[kDimsPerLane];
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) y[i] = x[i] * rstd * w[i] + bb[i];
  // Rotary pairs (2i, 2i+1): (a, b) -> (a c - b s, a s + b c). Identity
  // (c = 1, s = 0) past rope_dim, where it changes nothing.
  const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = y[2 * i], q = y[2 * i + 1];
    y[2 * i] = p * cc[i] - q * ss[i];
    y[2 * i + 1] = p * ss[i] + q * cc[i];
  }
  // Per-token scale from the largest magnitude.
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) m = fmaxf(m, fabsf(y[i]));
  const float amax = fmaxf(group_max(m), kAmaxFloor);
  const float inv = kE4M3Max / amax;
  int lo = 0, hi = 0;
  lo = cvt2_e4m3<false>(y[0] * inv, y[1] * inv, lo);
  lo = cvt2_e4m3<true>(y[2] * inv, y[3] * inv, lo);
  hi = cvt2_e4m3<false>(y[4] * inv, y[5] * inv, hi);
  hi = cvt2_e4m3<true>(y[6] * inv, y[7] * inv, hi);
  const int64_t slot = (int64_t)page * a.page_size + pos % a.page_size;
  if (page < 0 || slot >= a.num_slots) {
    if (sub == 0 && a.status) atomicOr(a.status, INDEXER_DEVICE_BAD_SLOT);
    return;
  }
  *reinterpret_cast<uint2*>(a.cache_fp8 + slot * kKeyDim + sub * kDimsPerLane) =
      make_uint2((uint32_t)lo, (uint32_t)hi);
  if (sub == 0) a.cache_scale[slot] = amax / kE4M3Max;
}

// Each 16-lane group takes kTokensPerGroup consecutive tokens and issues the
// loads of all of them before using any: the activations (addressed by the
// token index alone) go out with the token's position and row, and only
// the table entry and rotary row wait for those; then the arithmetic.
__global__ void __launch_bounds__(kPrologueBlock) key_prologue_kernel(KeyArgs a) {
  const int sub = (int)(threadIdx.x & (kLanesPerToken - 1));
  const int64_t tok0 = ((int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x / kLanesPerToken)) * kTokensPerGroup;
  int32_t row[kTokensPerGroup], pos[kTokensPerGroup];
  bool live[kTokensPerGroup];
  uint4 raw[kTokensPerGroup];
#pragma unroll
  for (int u = 0; u < kTokensPerGroup; ++u) {
    const int64_t tok = tok0 + u;
    const bool in = tok < a.num_tokens;
    row[u] = in ? (a.token_row ? a.token_row[tok] : 0) : -1;
    pos[u] = in ? a.positions[tok] : 0;
    raw[u] = in ? *reinterpret_cast<const uint4*>(a.k_act + tok * a.k_stride + sub * kDimsPerLane)
                : make_uint4(0u, 0u, 0u, 0u);
  }
  // (every test below is uniform over the token's 16 lanes)
#pragma unroll
  for (int u = 0; u < kTokensPerGroup; ++u) {
    live[u] = row[u] >= 0;   // a negative row is a padding token (or past the end)
    if (live[u] && (pos[u] < 0 || pos[u] >= a.max_pos)) {
      if (sub == 0 && a.status) atomicOr(a.status, INDEXER_DEVICE_BAD_POSITION);
      live[u] = false;
    }
  }
  const float4 w0 = *reinterpret_cast<const float4*>(a.weight + sub * kDimsPerLane);
  const float4 w1 = *reinterpret_cast<const float4*>(a.weight + sub * kDimsPerLane + 4);
  const float4 b0 = *reinterpret_cast<const float4*>(a.bias + sub * kDimsPerLane);
  const float4 b1 = *reinterpret_cast<const float4*>(a.bias + sub * kDimsPerLane + 4);
  const bool rot = sub * kDimsPerLane < a.rope_dim;   // this lane's 4 pairs are rotated
  int32_t page[kTokensPerGroup];
  float4 c[kTokensPerGroup], s[kTokensPerGroup];
#pragma unroll
  for (int u = 0; u < kTokensPerGroup; ++u) {
    page[u] = 0;
    c[u] = make_float4(1.f, 1.f, 1.f, 1.f);
    s[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live[u]) {
      page[u] = a.table[(int64_t)row[u] * a.table_stride + pos[u] / a.page_size];
      if (rot) {
        const float* cs = a.cos_sin + (int64_t)pos[u] * a.rope_dim + sub * (kDimsPerLane / 2);
        c[u] = *reinterpret_cast<const float4*>(cs);
        s[u] = *reinterpret_cast<const float4*>(cs + a.rope_dim / 2);
      }
    }
  }
  const float w[kDimsPerLane] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const float bb[kDimsPerLane] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
  for (int u = 0; u < kTokensPerGroup; ++u)
    if (live[u]) key_token(a, sub, pos[u], page[u], raw[u], w, bb, c[u], s[u]);
}

// Query path: rotary, per-(token, head) FP8 E4M3 and the head-gate weight
// with the query scale folded in. Same lane layout as the key path: 16 lanes
// per (token, head) row of 128 dims.
struct QueryArgs {
  const uint16_t* q;        // [T][H][128] BF16 bits
  int32_t rows;             // T * H
  int32_t heads;
  const float* w_raw;       // [T][H]
  float gate_scale;
  const float* cos_sin;
  int32_t rope_dim;
  int32_t max_pos;
  const int32_t* positions; // [T]
  uint8_t* q_codes;         // [T][H][128]
  float* w_out;             // [T][H]
  int32_t* status;
};

__global__ void __launch_bounds__(kPrologueBlock) query_prologue_kernel(QueryArgs a) {
  const int sub = (int)(threadIdx.x & (kLanesPerToken - 1));
  const int64_t r = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x / kLanesPerToken);
  if (r >= a.rows) return;   // (uniform over the row's 16 lanes)
  // (the codes and the gate weight go out with the position; only the
  // rotary row waits for it)
  const int32_t pos = a.positions[r / a.heads];
  const uint4 raw = *reinterpret_cast<const uint4*>(a.q + r * kKeyDim + sub * kDimsPerLane);
  const float w_raw = sub == 0 ? a.w_raw[r] : 0.f;
  const bool rot = sub * kDimsPerLane < a.rope_dim;
  if (a.rope_dim > 0 && (pos < 0 || pos >= a.max_pos)) {
    if (sub == 0 && a.status) atomicOr(a.status, INDEXER_DEVICE_BAD_POSITION);
    return;
  }
  float4 c = make_float4(1.f, 1.f, 1.f, 1.f), s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (rot) {
    const float* cs = a.cos_sin + (int64_t)pos * a.rope_dim + sub * (kDimsPerLane / 2);
    c = *reinterpret_cast<const float4*>(cs);
    s = *reinterpret_cast<const float4*>(cs + a.rope_dim / 2);
  }
  const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
  float y[kDimsPerLane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = __uint_as_float(words[i] << 16);
    y[2 * i + 1] = __uint_as_float(words[i] & 0xFFFF0000u);
  }
  const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = y[2 * i], q = y[2 * i + 1];
    y[2 * i] = p * cc[i] - q * ss[i];
    y[2 * i + 1] = p * ss[i] + q * cc[i];
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) m = fmaxf(m, fabsf(y[i]));
  const float amax = fmaxf(group_max(m), kAmaxFloor);
  const float inv = kE4M3Max / amax;
  int lo = 0, hi = 0;
  lo = cvt2_e4m3<false>(y[0] * inv, y[1] * inv, lo);
  lo = cvt2_e4m3<true>(y[2] * inv, y[3] * inv, lo);
  hi = cvt2_e4m3<false>(y[4] * inv, y[5] * inv, hi);
  hi = cvt2_e4m3<true>(y[6] * inv, y[7] * inv, hi);
  *reinterpret_cast<uint2*>(a.q_codes + r * kKeyDim + sub * kDimsPerLane) = make_uint2((uint32_t)lo, (uint32_t)hi);
  if (sub == 0) {
    const float q_scale = amax / kE4M3Max;
    a.w_out[r] = (w_raw * q_scale) * a.gate_scale;
  }
}

__global__ void debug_fp8_kernel(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (uint8_t)(cvt2_e4m3<false>(x[i], 0.f, 0) & 0xFF);
}

}  // namespace
}  // namespace satopk

using namespace satopk;

extern "C" {

topk_status indexer_key_prologue(const indexer_key_config* cfg, const uint16_t* k_act, int64_t k_stride,
                                 int32_t num_tokens, const float* ln_weight, const float* ln_bias,
                                 const float* cos_sin, const int32_t* positions, const int32_t* token_row,
                                 const int32_t* block_table, int64_t bt_row_stride, uint8_t* cache_fp8,
                                 float* cache_scale, int64_t num_slots, int32_t* status, void* stream) {
  if (!cfg || cfg->dim != kKeyDim || cfg->rope_dim < 0 || cfg->rope_dim > kKeyDim || cfg->rope_dim % 8 != 0 ||
      cfg->page_size < 1 || cfg->max_pos < 1 || !(cfg->eps >= 0.f) || !(cfg->eps < 3.0e38f))
    return TOPK_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (cfg->reserved[i] != 0) return TOPK_ERR_INVALID_ARG;
  if (num_tokens < 0 || k_stride < kKeyDim || k_stride % 8 != 0 || bt_row_stride < 0 || num_slots < 1)
    return TOPK_ERR_INVALID_ARG;
  if (num_tokens == 0) return TOPK_OK;
  if (!k_act || !ln_weight || !ln_bias || !positions || !block_table || !cache_fp8 || !cache_scale)
    return TOPK_ERR_INVALID_ARG;
  if (cfg->rope_dim > 0 && !cos_sin) return TOPK_ERR_INVALID_ARG;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (misaligned(k_act) || misaligned(ln_weight) || misaligned(ln_bias) || misaligned(cache_fp8) ||
      (cfg->rope_dim > 0 && misaligned(cos_sin)))
    return TOPK_ERR_INVALID_ARG;
  KeyArgs a;
  a.k_act = k_act;
  a.k_stride = k_stride;
  a.num_tokens = num_tokens;
  a.weight = ln_weight;
  a.bias = ln_bias;
  a.eps = cfg->eps;
  a.cos_sin = cos_sin;
  a.rope_dim = cfg->rope_dim;
  a.max_pos = cfg->max_pos;
  a.positions = positions;
  a.token_row = token_row;
  a.table = block_table;
  a.table_stride = bt_row_stride;
  a.page_size = cfg->page_size;
  a.cache_fp8 = cache_fp8;
  a.cache_scale = cache_scale;
  a.num_slots = num_slots;
  a.status = status;   // may be NULL: the flags are then dropped
  const unsigned blocks = (unsigned)((num_tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(key_prologue_kernel, dim3(blocks), dim3(kPrologueBlock), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

topk_status indexer_query_prologue(const uint16_t* q_act, int32_t tokens, int32_t heads, const float* w_raw,
                                   float gate_scale, const float* cos_sin, int32_t rope_dim, int32_t max_pos,
                                   const int32_t* positions, uint8_t* q_codes, float* w_out, int32_t* status,
                                   void* stream) {
  if (tokens < 0 || heads < 1 || rope_dim < 0 || rope_dim > kKeyDim || rope_dim % 8 != 0 || max_pos < 1 ||
      !(gate_scale > 0.f) || !(gate_scale < 3.0e38f) || (int64_t)tokens * heads > 0x7FFFFFFF)
    return TOPK_ERR_INVALID_ARG;
  if (tokens == 0) return TOPK_OK;
  if (!q_act || !w_raw || !positions || !q_codes || !w_out || (rope_dim > 0 && !cos_sin)) return TOPK_ERR_INVALID_ARG;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (misaligned(q_act) || misaligned(q_codes) || (rope_dim > 0 && misaligned(cos_sin))) return TOPK_ERR_INVALID_ARG;
  QueryArgs a;
  a.q = q_act;
  a.rows = tokens * heads;
  a.heads = heads;
  a.w_raw = w_raw;
  a.gate_scale = gate_scale;
  a.cos_sin = cos_sin;
  a.rope_dim = rope_dim;
  a.max_pos = max_pos;
  a.positions = positions;
  a.q_codes = q_codes;
  a.w_out = w_out;
  a.status = status;
  const unsigned blocks = (unsigned)((a.rows + kGroupsPerBlock - 1) / kGroupsPerBlock);
  hipLaunchKernelGGL(query_prologue_kernel, dim3(blocks), dim3(kPrologueBlock), 0, static_cast<hipStream_t>(stream),
                     a);
  return hipGetLastError() == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

topk_status indexer_debug_fp8(const float* x, int64_t n, uint8_t* out, void* stream) {
  if (n < 0 || (n > 0 && (!x || !out))) return TOPK_ERR_INVALID_ARG;
  if (n == 0) return TOPK_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(debug_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), x,
                     n, out);
  return hipGetLastError() == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

}  // extern "C"
