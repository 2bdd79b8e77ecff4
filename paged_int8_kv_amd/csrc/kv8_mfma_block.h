// Per-block arithmetic of the matrix-core decode kernels of libkv8 on
// gfx950 (kv8_decode_mfma.hip: the one-pass and two-pass split kernels;
// kv8_decode_sk.hip: the stream-K kernel): q as the B operand of the logit
// MFMAs, the logit MFMA's A operand from a block's K codes, the value MFMAs
// of a block's V codes, and the row-wise max across the four 16-lane rows.
// The operand layouts are described at the top of kv8_decode_mfma.hip.
// Nothing here is used outside the HIP library.
#pragma once

#include "kv8_decode_common.h"
#include "kv8_device.h"

namespace kv8 {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8_t cat8(half2_t a, half2_t b, half2_t c, half2_t d) {
  const half4_t lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const half4_t hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ half4_t cat4(half2_t a, half2_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3);
}
__device__ __forceinline__ uint32_t dw(const uint4& r, int k) {
  return k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w;
}

// Max over the four rows of 16 lanes (lanes l, l^16, l^32, l^48), every lane
// receiving it: two row swaps on the vector unit, no LDS crossbar.
__device__ __forceinline__ float rows_max(float x) {
  float a, b;
  swap16(x, a, b);
  x = fmaxf(a, b);
  swap32(x, a, b);
  return fmaxf(a, b);
}

// Nontemporal loads of cache codes, for kernels that stream every code once
// over a footprint larger than the last-level cache.
typedef unsigned int ntu32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int ntu32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  const ntu32x4 v = __builtin_nontemporal_load(reinterpret_cast<const ntu32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 nt_load(const uint2* p) {
  const ntu32x2 v = __builtin_nontemporal_load(reinterpret_cast<const ntu32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t nt_load(const uint32_t* p) {
  return __builtin_nontemporal_load(p);
}

template <int NDW> struct VRowT;
template <> struct VRowT<2> { using type = uint2; };
template <> struct VRowT<1> { using type = uint32_t; };
__device__ __forceinline__ uint32_t dw(const uint2& r, int k) { return k == 0 ? r.x : r.y; }
__device__ __forceinline__ uint32_t dw(const uint32_t& r, int) { return r; }

// q of head hl (lane % 16; zero for hl >= G) as the B operands of the logit
// MFMAs: for MFMA j the 8 channels 64(j/2) + 16 q4 + 8(j%2) ... + 7 of byte
// codes, or for 4-bit codes the channels 32 q4 + 8j + (0, 4, 1, 5, 2, 6, 3,
// 7) in the order the nibble pairs come out, in fp16
// after the head's power-of-two rescale (bf16 q is exact then; an fp32 q
// also gets its fp16 remainder in qlo).  cz = log2(e) * sm_scale undoing the
// rescale and the K codes' value step; nqb = minus the K codes' logit bias
// times the head's fp16 q sum (the logit accumulators start there).
template <int D, int G, bool QF32, class C>
__device__ __forceinline__ void q_operands(const SplitArgs& a, int64_t bh0, int hl, int q4,
                                           half8_t (&qb)[D / 32],
                                           half8_t (&qlo)[QF32 ? D / 32 : 1], float& cz,
                                           float& nqb) {
  constexpr int NKM = D / 32;
  constexpr bool NIB = C::kBits == 4;
  const bool live = hl < G;
  const int64_t qrow = (bh0 + (live ? hl : 0)) * D;
  float x[NKM][8];
#pragma unroll
  for (int j = 0; j < NKM; ++j) {
    const int c0 = NIB ? 32 * q4 + 8 * j : 64 * (j / 2) + 16 * q4 + 8 * (j % 2);
    if constexpr (QF32) {
      const float4* qp = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qrow + c0);
      const float4 u = qp[0], v = qp[1];
      x[j][0] = u.x; x[j][1] = u.y; x[j][2] = u.z; x[j][3] = u.w;
      x[j][4] = v.x; x[j][5] = v.y; x[j][6] = v.z; x[j][7] = v.w;
    } else {
      const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qrow + c0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = dw(r, k);
        x[j][2 * k] = __builtin_bit_cast(float, w << 16);
        x[j][2 * k + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) x[j][i] = live ? x[j][i] : 0.0f;
    if constexpr (NIB) {   // slot order of the nibble pairs: channels 0,4,1,5,2,6,3,7
      const float y[8] = {x[j][0], x[j][4], x[j][1], x[j][5], x[j][2], x[j][6], x[j][3], x[j][7]};
#pragma unroll
      for (int i = 0; i < 8; ++i) x[j][i] = y[i];
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < NKM; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[j][i]));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  // power-of-two shift bringing the head's largest |q| into [2^14, 2^15)
  const int e = m > 0.0f ? ilogbf(m) - 14 : 0;
  float qsum = 0.0f;
#pragma unroll
  for (int j = 0; j < NKM; ++j) {
    _Float16 hv[8], lv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sc = ldexpf(x[j][i], -e);
      hv[i] = (_Float16)sc;
      qsum += (float)hv[i];
      if constexpr (QF32) {
        lv[i] = (_Float16)(sc - (float)hv[i]);
        qsum += (float)lv[i];
      }
    }
    qb[j] = half8_t{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
    if constexpr (QF32) qlo[j] = half8_t{lv[0], lv[1], lv[2], lv[3], lv[4], lv[5], lv[6], lv[7]};
  }
  qsum += __shfl_xor(qsum, 16);
  qsum += __shfl_xor(qsum, 32);
  cz = ldexpf(a.qk_scale_log2, e) * (1.0f / C::kLogitStep);
  nqb = -C::kLogitBias * qsum;
}

// The logit MFMA's A operand j of a block: the lane's 8 channels of MFMA j
// (the same channels q_operands puts in B).  Byte codes: dwords 2(j%2) and
// 2(j%2)+1 of 16-byte piece j/2.  4-bit codes: dword j of the lane's single
// 16-byte piece, as nibble pairs (c, c+4).
template <class C, int NCH>
__device__ __forceinline__ half8_t logit_operand(const uint4 (&rk)[NCH], int j) {
  if constexpr (C::kBits == 4) {
    const uint32_t x = dw(rk[0], j);
    return cat8(C::logit_pair_raw(x, 0), C::logit_pair_raw(x, 1), C::logit_pair_raw(x, 2),
                C::logit_pair_raw(x, 3));
  } else {
    const uint4 r = rk[j / 2];
    const uint32_t x0 = C::pre(dw(r, 2 * (j % 2))), x1 = C::pre(dw(r, 2 * (j % 2) + 1));
    return cat8(C::lo(x0), C::hi(x0), C::lo(x1), C::hi(x1));
  }
}

// The value MFMAs of a block: acc[j] += A_j . wb with A_j the codes of
// channel (D/16) hl + j for the 4 tokens whose rows the lane holds.  Byte
// codes: one interleave per token pair and dword, then byte pairs.  4-bit
// codes (D = 128): the 4 tokens' dwords hold channels 8 hl .. + 7; one byte
// permute joins two tokens' low (high) halves, whose nibble pairs are then
// (token t, token t+1) of channel j (4 + j).  INT8 codes (c + 1152) are
// unbiased here, exactly, by one packed fp16 subtract per pair: summing
// biased codes over a long split and taking bias * sum(w) off at its end
// cancels away too many bits (measured at 264K tokens: INT8 7.3e-4, INT4
// with a bias of 1032 1.5e-3, against 2.1e-4 unbiased).  INT4 codes enter
// as 1.5 + c/16, a bias of 24 code steps, and leave it through the weight
// sums accw (one more MFMA per block, value_unbias at the end; 258K INT4
// relative error 6.3e-5) in place of the 16 subtracts per block.

template <class C, int NVT, class VRow>
__device__ __forceinline__ void value_mfmas(const VRow (&rv)[4], half4_t wb,
                                            float4_t (&acc)[NVT], float4_t& accw) {
  if constexpr (C::kBits == 4) {
    const uint32_t u0 = dw(rv[0], 0), u1 = dw(rv[1], 0);
    const uint32_t u2 = dw(rv[2], 0), u3 = dw(rv[3], 0);
    const uint32_t l01 = __builtin_amdgcn_perm(u1, u0, 0x05040100u);
    const uint32_t h01 = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    const uint32_t l23 = __builtin_amdgcn_perm(u3, u2, 0x05040100u);
    const uint32_t h23 = __builtin_amdgcn_perm(u3, u2, 0x07060302u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(
          cat4(C::value_pair_raw(l01, j), C::value_pair_raw(l23, j)), wb, acc[j], 0, 0, 0);
      acc[4 + j] = __builtin_amdgcn_mfma_f32_16x16x16f16(
          cat4(C::value_pair_raw(h01, j), C::value_pair_raw(h23, j)), wb, acc[4 + j], 0, 0, 0);
    }
    // the weight sums of the 4 tokens per head, for value_unbias
    const half4_t ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
    accw = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, wb, accw, 0, 0, 0);
  } else {
#pragma unroll
    for (int k = 0; k < NVT / 4; ++k) {
      const uint32_t x0 = C::pre(dw(rv[0], k)), x1 = C::pre(dw(rv[1], k));
      const uint32_t x2 = C::pre(dw(rv[2], k)), x3 = C::pre(dw(rv[3], k));
      const uint32_t l01 = interleave_lo(x0, x1), h01 = interleave_hi(x0, x1);
      const uint32_t l23 = interleave_lo(x2, x3), h23 = interleave_hi(x2, x3);
      const half4_t t0 = cat4(C::exact(C::lo(l01)), C::exact(C::lo(l23)));   // byte 4k
      const half4_t t1 = cat4(C::exact(C::hi(l01)), C::exact(C::hi(l23)));   // byte 4k+1
      const half4_t t2 = cat4(C::exact(C::lo(h01)), C::exact(C::lo(h23)));   // byte 4k+2
      const half4_t t3 = cat4(C::exact(C::hi(h01)), C::exact(C::hi(h23)));   // byte 4k+3
      acc[4 * k] = __builtin_amdgcn_mfma_f32_16x16x16f16(t0, wb, acc[4 * k], 0, 0, 0);
      acc[4 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(t1, wb, acc[4 * k + 1], 0, 0, 0);
      acc[4 * k + 2] = __builtin_amdgcn_mfma_f32_16x16x16f16(t2, wb, acc[4 * k + 2], 0, 0, 0);
      acc[4 * k + 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(t3, wb, acc[4 * k + 3], 0, 0, 0);
    }
  }
}

// The accumulators as sums of w * c: 4-bit value codes enter value_mfmas as
// kValueBias + c * kValueStep, which value_unbias takes off through the
// weight sums accw (byte codes enter exact and are left as they are).
template <class C, int NVT>
__device__ __forceinline__ void value_unbias(float4_t (&acc)[NVT], const float4_t& accw) {
  if constexpr (C::kBits == 4) {
    constexpr float inv = 1.0f / C::kValueStep;
#pragma unroll
    for (int j = 0; j < NVT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[j][r] = acc[j][r] * inv - (C::kValueBias * inv) * accw[r];
  }
}

}  // namespace

}  // namespace kv8
