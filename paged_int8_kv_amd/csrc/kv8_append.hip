// kv8_quant_append kernel: per-token, per-KV-head quantisation of new K/V
// rows to INT8 (or to FP8 e4m3, or to nibble-packed INT4, for those caches)
// and their scatter into 16-token physical blocks.
//
// The method keeps K/V as INT8 produced by dynamic per-token quantisation
// ("KV-Cache 全栈优化系统" README, section 主要特性); slots address physical
// blocks through the block table ("KV Cache 优化全景解析", section 4.2).
//
// Work mapping: one row = (token n, KV head h) of length d.  LPR = d / 8
// lanes share a row, each lane holding 8 bf16 values (one 16-byte load) of
// K and the same 8 of V.  The absmax is reduced across the LPR lanes with
// DPP; the fp32 scale is divided with IEEE-correct division (hipcc's
// default), rounded to fp16 (round-to-nearest-even, subnormals kept) and
// saturated to 65504; codes use IEEE division, then v_rndne (ties to even)
// and a symmetric clamp for INT8 (and INT4), or round-to-nearest-even on
// the e4m3 grid with saturation for FP8 (the code formats are described in
// kv8_device.h).  Each lane stores its 8 codes (8 bytes; 4 for INT4) so
// that the LPR lanes write one contiguous row of the block.
#include "kv8_device.h"
#include "kv8_launch.h"

namespace kv8 {

namespace {


// Rotary embedding of K (rotate-half convention over the whole head): for
// j < d/2 with (c, s) = cos_sin[pos][j], cos_sin[pos][d/2 + j],
//   x'_j = x_j c - x_{j+d/2} s,   x'_{j+d/2} = x_{j+d/2} c + x_j s,
// each product and the sum rounded to fp32 (contraction off), so the
// quantiser sees the same fp32 values as any plain implementation.  The
// lane holding channels j and the lane holding j + d/2 are LPR/2 apart in
// the row, so one lane exchange per value brings the partner over.
template <int LPR>
__device__ __forceinline__ void rope8(float (&x)[8], int part, const float* __restrict__ cs,
                                      int half) {
#pragma clang fp contract(off)
  const bool upper = part >= LPR / 2;
  const int j0 = (part % (LPR / 2)) * 8;            // first channel index within the half
  const float4 c0 = *reinterpret_cast<const float4*>(cs + j0);
  const float4 c1 = *reinterpret_cast<const float4*>(cs + j0 + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(cs + half + j0);
  const float4 s1 = *reinterpret_cast<const float4*>(cs + half + j0 + 4);
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __shfl_xor(x[i], LPR / 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = x[i] * c[i];
    const float b = p[i] * sn[i];
    x[i] = upper ? a + b : a - b;
  }
}

template <int D, class C, bool ROPE>
__global__ __launch_bounds__(256) void quant_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slot_mapping, int64_t n_rows, int num_kv_heads,
    int64_t num_slots, int8_t* __restrict__ k_cache, int8_t* __restrict__ v_cache,
    uint16_t* __restrict__ k_scale, uint16_t* __restrict__ v_scale,
    const int32_t* __restrict__ positions, const float* __restrict__ cos_sin,
    int max_position) {
  constexpr int LPR = D / 8;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gtid / LPR;          // (token, head) row
  const int part = (int)(gtid % LPR);      // which 8 channels
  if (row >= n_rows) return;               // whole rows exit together
  // rows fit 31 bits (checked on the host): 32-bit division by the head count
  const uint32_t row32 = (uint32_t)row, nh = (uint32_t)num_kv_heads;
  const uint32_t n = row32 / nh;
  const int h = (int)(row32 - n * nh);
  const int64_t slot = slot_mapping[n];
  const bool keep = slot >= 0 && slot < num_slots;

  // K and V are read once: nontemporal loads (fill 185 -> 153 us per call
  // for 131,072 tokens x 8 heads; nontemporal code stores measured slower)
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 kv4 =
      __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_new + row * D + part * 8));
  const u32x4 vv4 =
      __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_new + row * D + part * 8));
  const uint4 kraw = make_uint4(kv4.x, kv4.y, kv4.z, kv4.w);
  const uint4 vraw = make_uint4(vv4.x, vv4.y, vv4.z, vv4.w);
  float kx[8], vx[8], ka, va;
  unpack8(kraw, kx, ka);
  unpack8(vraw, vx, va);
  if constexpr (ROPE) {
    int pos = positions[n];
    pos = pos < 0 ? 0 : (pos >= max_position ? max_position - 1 : pos);
    rope8<LPR>(kx, part, cos_sin + (int64_t)pos * D, D / 2);
    ka = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ka = fmaxf(ka, fabsf(kx[i]));
  }
  // Every lane of the row takes part in the reductions (rows never straddle
  // an exit), so the DPP partners are always active.
  ka = row_absmax<LPR>(ka);
  va = row_absmax<LPR>(va);
  if (!keep) return;

  const float ks = fp16_scale<C>(ka);
  const float vs = fp16_scale<C>(va);
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot % kBlock);
  const int64_t line = (blk * num_kv_heads + h) * kBlock + off;   // (block, head, slot)
  if constexpr (C::kBits == 4) {
    *reinterpret_cast<uint32_t*>(k_cache + line * (D / 2) + part * 4) =
        quantise8_nibbles<C>(kx, ks);
    *reinterpret_cast<uint32_t*>(v_cache + line * (D / 2) + part * 4) =
        quantise8_nibbles<C>(vx, vs);
  } else {
    *reinterpret_cast<uint2*>(k_cache + line * D + part * 8) = quantise8<C>(kx, ks);
    *reinterpret_cast<uint2*>(v_cache + line * D + part * 8) = quantise8<C>(vx, vs);
  }
  if (part == 0) {
    k_scale[line] = __builtin_bit_cast(uint16_t, (_Float16)ks);
    v_scale[line] = __builtin_bit_cast(uint16_t, (_Float16)vs);
  }
}

}  // namespace

namespace {
template <class C, bool ROPE>
void launch_append_fmt(const uint16_t* k_new, const uint16_t* v_new, const int32_t* slot_mapping,
                       int64_t n_rows, int num_kv_heads, int head_dim, int64_t num_slots,
                       int8_t* k_cache, int8_t* v_cache, uint16_t* k_scale, uint16_t* v_scale,
                       const int32_t* positions, const float* cos_sin, int max_position,
                       hipStream_t stream) {
  const int64_t threads = n_rows * (head_dim / 8);
  const int64_t grid = (threads + 255) / 256;
  if (head_dim == 128) {
    quant_append_kernel<128, C, ROPE><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
        k_new, v_new, slot_mapping, n_rows, num_kv_heads, num_slots, k_cache, v_cache,
        k_scale, v_scale, positions, cos_sin, max_position);
  } else {
    quant_append_kernel<64, C, ROPE><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
        k_new, v_new, slot_mapping, n_rows, num_kv_heads, num_slots, k_cache, v_cache,
        k_scale, v_scale, positions, cos_sin, max_position);
  }
}
}  // namespace

int launch_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                        const int32_t* slot_mapping, int64_t n_tokens, int num_kv_heads,
                        int head_dim, int64_t num_blocks, int8_t* k_cache, int8_t* v_cache,
                        uint16_t* k_scale, uint16_t* v_scale, int fmt, hipStream_t stream) {
  const int64_t n_rows = n_tokens * num_kv_heads;
  const int64_t num_slots = num_blocks * kBlock;
  if (fmt == kFmtInt4)
    launch_append_fmt<CodesInt4, false>(k_new, v_new, slot_mapping, n_rows, num_kv_heads,
                                        head_dim, num_slots, k_cache, v_cache, k_scale, v_scale,
                                        nullptr, nullptr, 0, stream);
  else if (fmt == kFmtFp8)
    launch_append_fmt<CodesFp8, false>(k_new, v_new, slot_mapping, n_rows, num_kv_heads,
                                       head_dim, num_slots, k_cache, v_cache, k_scale, v_scale,
                                       nullptr, nullptr, 0, stream);
  else
    launch_append_fmt<CodesInt8, false>(k_new, v_new, slot_mapping, n_rows, num_kv_heads,
                                        head_dim, num_slots, k_cache, v_cache, k_scale, v_scale,
                                        nullptr, nullptr, 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_rope_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                             const int32_t* slot_mapping, const int32_t* positions,
                             const float* cos_sin, int max_position, int64_t n_tokens,
                             int num_kv_heads, int head_dim, int64_t num_blocks, int8_t* k_cache,
                             int8_t* v_cache, uint16_t* k_scale, uint16_t* v_scale,
                             hipStream_t stream) {
  launch_append_fmt<CodesInt8, true>(k_new, v_new, slot_mapping, n_tokens * num_kv_heads,
                                     num_kv_heads, head_dim, num_blocks * kBlock, k_cache,
                                     v_cache, k_scale, v_scale, positions, cos_sin, max_position,
                                     stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
