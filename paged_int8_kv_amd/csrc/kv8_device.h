// Device-side helpers shared by the gfx950 kernels of libkv8.
//
// Cross-lane primitives (DPP, permlane swaps), byte permutes and the
// int8 -> fp16 conversion used by the attention kernels.  Nothing here is
// used outside the HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kv8 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;          // tokens per physical block
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// DPP lane exchanges inside a 64-lane wave.  Control codes follow the GCN /
// CDNA DPP encoding: quad_perm(a,b,c,d) = a | b<<2 | c<<4 | d<<6,
// row_ror:n = 0x120 + n, row_mirror = 0x140, row_half_mirror = 0x141.
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadXor1 = 0xB1,       // [1,0,3,2]
  kDppQuadXor2 = 0x4E,       // [2,3,0,1]
  kDppHalfMirror = 0x141,    // lane i <-> 7-i inside each group of 8
  kDppRowMirror = 0x140,     // lane i <-> 15-i inside each row of 16
  kDppRowRor8 = 0x128,       // lane i <- (i+8) mod 16 inside each row
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum / max over aligned groups of 8 consecutive lanes; every lane of the
// group receives the result.  After the two quad steps all four lanes of a
// quad agree, so the half-mirror step adds the two quads of the group.
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_f<kDppQuadXor1>(x);
  x += dpp_f<kDppQuadXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x;
}
__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  return x;
}
__device__ __forceinline__ float group16_max(float x) {
  x = group8_max(x);
  x = fmaxf(x, dpp_f<kDppRowMirror>(x));
  return x;
}

// Row swaps: v_permlane16_swap exchanges rows 1,3 of its first operand with
// rows 0,2 of its second (x' = [x.r0, y.r0, x.r2, y.r2], y' = [x.r1, y.r1,
// x.r3, y.r3] for rows of 16 lanes); v_permlane32_swap exchanges the upper
// half of the first with the lower half of the second (x' = [x.lo, y.lo],
// y' = [x.hi, y.hi]).  Written as inline asm with both operands read-write:
// through the builtin, the compiler used the first result twice when the
// two results were added.  The leading s_nop covers the VALU-write ->
// permlane-read wait states.
__device__ __forceinline__ void swap16_pair(float x, float y, float& xo, float& yo) {
  float u = x, v = y;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(u), "+v"(v));
  xo = u;
  yo = v;
}
__device__ __forceinline__ void swap32_pair(float x, float y, float& xo, float& yo) {
  float u = x, v = y;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(u), "+v"(v));
  xo = u;
  yo = v;
}
__device__ __forceinline__ void swap16(float x, float& a, float& b) { swap16_pair(x, x, a, b); }
__device__ __forceinline__ void swap32(float x, float& a, float& b) { swap32_pair(x, x, a, b); }

// Sum of the eight lanes {l, l^8, l^16, ..., l^56} (same position inside
// every group of 8); every lane receives the sum of its class.
__device__ __forceinline__ float across_groups_sum(float x) {
  float a, b;
  x += dpp_f<kDppRowRor8>(x);
  swap16(x, a, b);
  x = a + b;
  swap32(x, a, b);
  return a + b;
}
__device__ __forceinline__ float across_groups_max(float x) {
  float a, b;
  x = fmaxf(x, dpp_f<kDppRowRor8>(x));
  swap16(x, a, b);
  x = fmaxf(a, b);
  swap32(x, a, b);
  return fmaxf(a, b);
}

// ---------------------------------------------------------------------------
// int8 codes -> fp16 pairs without a convert instruction per code.
// A code c becomes the byte u = c + 128 (xor 0x80); placing u under the fp16
// high byte 0x64 gives the fp16 value 1024 + u = c + 1152 exactly.  Dot
// products therefore carry a bias of 1152 * (sum of the other operand),
// which the kernels subtract once per token or per output.
// v_perm_b32 selector bytes 0-3 pick bytes of the second operand, 4-7
// bytes of the first.
// ---------------------------------------------------------------------------
constexpr uint32_t kXor80 = 0x80808080u;
constexpr uint32_t kHi64 = 0x64646464u;
constexpr float kCodeBias = 1152.0f;

__device__ __forceinline__ half2_t biased_pair_lo(uint32_t u) {   // bytes 0,1
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(kHi64, u, 0x04010400u));
}
__device__ __forceinline__ half2_t biased_pair_hi(uint32_t u) {   // bytes 2,3
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(kHi64, u, 0x04030402u));
}
// Interleave bytes k, k+1 of two words: [a.k, b.k, a.k+1, b.k+1].
__device__ __forceinline__ uint32_t interleave_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05010400u);
}
__device__ __forceinline__ uint32_t interleave_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07030602u);
}

__device__ __forceinline__ float fdot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// ---------------------------------------------------------------------------
// Code formats of the quantised cache.  Each holds one code per byte, a
// per-(token, KV head) fp16 scale and the quantiser's largest code value:
//   CodesInt8  symmetric INT8, codes -127..127 (the KV8 method);
//   CodesFp8   OCP e4m3 ("KV Cache 优化全景解析", section 7.4), largest 448.
// pre() + lo()/hi() turn a dword of 4 codes into two fp16 pairs (bytes 0,1
// and 2,3).  For INT8 the pairs carry the +1152 bias described above;
// exact() removes it.  e4m3 values are all exact in fp16, so the FP8 pairs
// come from one hardware convert each and need no bias (exact() is the
// identity).  The decode kernels feed K codes to the logit products as the
// values kLogitBias + kLogitStep * c and start each sum at minus kLogitBias
// * sum(q); the logit scale absorbs 1 / kLogitStep (a power of two).  The
// cancellation this leaves costs an INT8 logit about 3e-5 (log2 units) at
// most.
// code() quantises one value: the fp32 quotient x / s (IEEE division), then
// INT8: round half to even and clamp to +-127; FP8: round to nearest even
// on the e4m3 grid and saturate to +-448, the sign of a zero kept.
// ---------------------------------------------------------------------------
struct CodesInt8 {
  static constexpr int kBits = 8;
  static constexpr bool kIntCodes = true;   // code = clamp(rint(quotient))
  static constexpr float kBias = kCodeBias;
  static constexpr float kLogitBias = kCodeBias;
  static constexpr float kLogitStep = 1.0f;
  static constexpr float kQmax = 127.0f;
  __device__ static uint32_t pre(uint32_t u) { return u ^ kXor80; }
  __device__ static half2_t lo(uint32_t x) { return biased_pair_lo(x); }
  __device__ static half2_t hi(uint32_t x) { return biased_pair_hi(x); }
  __device__ static half2_t exact(half2_t p) {
    const half2_t bias = {(_Float16)kCodeBias, (_Float16)kCodeBias};
    return p - bias;
  }
  __device__ static uint32_t code_of_quotient(float q) {   // q = fl32(x / s)
    float c = __builtin_rintf(q);                      // ties to even
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    return (uint32_t)((int32_t)c) & 0xFFu;
  }
  __device__ static uint32_t code(float x, float s) {
    return code_of_quotient(x / s);                   // IEEE divide
  }
};

struct CodesFp8 {
  static constexpr int kBits = 8;
  static constexpr bool kIntCodes = false;
  static constexpr float kBias = 0.0f;
  static constexpr float kLogitBias = 0.0f;
  static constexpr float kLogitStep = 1.0f;
  static constexpr float kQmax = 448.0f;
  __device__ static uint32_t pre(uint32_t u) { return u; }
  __device__ static half2_t lo(uint32_t x) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  }
  __device__ static half2_t hi(uint32_t x) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  }
  __device__ static half2_t exact(half2_t p) { return p; }
  __device__ static uint32_t code(float x, float s) {
    const float q = x / s;                            // IEEE divide
    const uint32_t sign = (__builtin_bit_cast(uint32_t, q) >> 24) & 0x80u;
    const float a = fabsf(q);
    uint32_t c;
    if (a >= 448.0f) {
      c = 0x7Eu;                                      // 448; beyond it saturates
    } else if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
      c = (uint32_t)__builtin_rintf(a * 512.0f);      // exact scaling, ties to even
    } else {                                          // 3 mantissa bits, ties to even
      const uint32_t ua = __builtin_bit_cast(uint32_t, a);
      c = ((ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20) - (120u << 3);
    }
    return sign | c;
  }
};

// INT4: symmetric codes -7..7 (the INT8 recipe with 7 in place of 127), two
// per byte as 4-bit two's complement, element 2i in the low nibble of byte
// i.  A dword holds 8 codes.  Flipping each nibble's sign bit (xor 0x8)
// gives u = c + 8, and u under the fp16 pattern 0x6400 is the value
// 1024 + u = c + 1032 exactly.  nib_pair(x, j) makes the fp16 pair of
// nibbles j and j + 4 of the (already flipped) dword x.  The logit pairs
// (logit_pair_raw) hold u in the top four mantissa bits under 0x3C00,
// the value 1 + u / 16 = 1.5 + c / 16 exactly, for the logit products: a
// bias of 24 code steps in place of 1032 (summed against q of up to 2^15,
// the 1032 bias cost the logits enough to put 6e-4 relative error into the
// output at 264K tokens), at the same two operations per pair.
struct CodesInt4 {
  static constexpr int kBits = 4;
  static constexpr bool kIntCodes = true;
  static constexpr float kBias = 1032.0f;
  static constexpr float kLogitBias = 1.5f;
  static constexpr float kLogitStep = 0.0625f;
  static constexpr float kQmax = 7.0f;
  __device__ static uint32_t pre(uint32_t u) { return u ^ 0x88888888u; }
  __device__ static half2_t nib_pair(uint32_t x, int j) {
    return __builtin_bit_cast(half2_t, ((x >> (4 * j)) & 0x000F000Fu) | 0x64006400u);
  }
  // The pairs from the raw dword, without pre(): the sign flip commutes
  // with the shift and the mask, and its bit meets none of the fp16
  // pattern's, so it folds into that constant; a pair is then one shift and
  // one three-input bit operation.
  __device__ static half2_t nib_pair_raw(uint32_t x, int j) {
    return __builtin_bit_cast(half2_t, ((x >> (4 * j)) & 0x000F000Fu) ^ 0x64086408u);
  }
  // The value operands use the logits' encoding, 1 + u/16 = kValueBias +
  // c * kValueStep: one shift and one bit-op per pair, no subtract; the
  // bias leaves once per split through the weight sums (value_unbias).
  static constexpr float kValueBias = 1.5f;
  static constexpr float kValueStep = 0.0625f;
  __device__ static half2_t value_pair_raw(uint32_t x, int j) { return logit_pair_raw(x, j); }
  __device__ static half2_t logit_pair_raw(uint32_t x, int j) {
    const uint32_t y = j < 2 ? x << (6 - 4 * j) : x >> (4 * j - 6);
    return __builtin_bit_cast(half2_t, (y & 0x03C003C0u) ^ 0x3E003E00u);
  }
  __device__ static half2_t exact(half2_t p) {
    const half2_t bias = {(_Float16)kBias, (_Float16)kBias};
    return p - bias;
  }
  __device__ static uint32_t code_of_quotient(float q) {   // q = fl32(x / s)
    float c = __builtin_rintf(q);                      // ties to even
    c = fminf(fmaxf(c, -7.0f), 7.0f);
    return (uint32_t)((int32_t)c) & 0xFu;
  }
  __device__ static uint32_t code(float x, float s) {
    return code_of_quotient(x / s);                   // IEEE divide
  }
};

// ---------------------------------------------------------------------------
// Row quantiser shared by the append kernel and the decode step that appends
// its newest token: LPR lanes hold one (token, KV head) row of d = 8 * LPR
// bf16 values, 8 per lane.  Scale s = fp16_rne(fp32(absmax / kQmax)) with
// gradual underflow, saturated to 65504; codes by C::code; a zero scale
// gives all-zero codes.
// ---------------------------------------------------------------------------
template <int LPR>
__device__ __forceinline__ float row_absmax(float a) {
  static_assert(LPR == 8 || LPR == 16, "row of 64 or 128 channels");
  if constexpr (LPR == 8) return group8_max(a);
  else return group16_max(a);
}

template <class C>
__device__ __forceinline__ float fp16_scale(float absmax) {
  const float s32 = absmax / C::kQmax;               // IEEE divide, RNE
  _Float16 s16 = (_Float16)s32;                       // RNE, gradual underflow
  if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
  return (float)s16;
}

// Integer codes rint(fl32(x / s)) of a lane's 8 values without a division
// per value where that is provably the same.  q_a = x * rcp(s) (v_rcp_f32,
// relative error <= 2^-23) differs from the specified fp32 quotient
// fl32(x / s) by at most about 2^-21.6 |q|, so both round to the same
// integer unless q_a lies within that distance of a half-integer; a lane
// with any value within 2^-20 |q_a| of one (every exact tie among them)
// takes the IEEE division for all 8.  Returns the quotients to round.
template <int N>
__device__ __forceinline__ void quotients(const float (&x)[N], float s, float (&q)[N]) {
  const float r = __builtin_amdgcn_rcpf(s);
  bool near = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    q[i] = x[i] * r;
    const float a = fabsf(q[i]);
    near |= fabsf(__builtin_amdgcn_fractf(a) - 0.5f) <= a * 0x1p-20f;   // fract: a - floor(a), exact
  }
  if (__builtin_expect(near, 0)) {
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = x[i] / s;   // IEEE divide
  }
}

// Integer code of a quotient as the low bits of an fp32: q clamped to
// [-qmax, qmax] (clamping to integer bounds commutes with rounding), plus
// 1.5 * 2^23, rounds to the nearest integer with ties to even (the fp32 add
// itself rounds so, the magic constant being even), and the sum's bits are
// 0x4B400000 + rint(q): their low byte (nibble) is the code in two's
// complement.
__device__ __forceinline__ uint32_t code_bits(float q, float qmax) {
  const float c = __builtin_amdgcn_fmed3f(q, -qmax, qmax);
  return __builtin_bit_cast(uint32_t, c + 12582912.0f);
}

template <class C>
__device__ __forceinline__ uint2 quantise8(const float (&x)[8], float s) {
  uint32_t w0 = 0, w1 = 0;
  if (s != 0.0f) {
    if constexpr (C::kIntCodes) {
      float q[8];
      quotients<8>(x, s, q);
      uint32_t y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = code_bits(q[i], C::kQmax);
      // low bytes of y0..y3 -> one dword: [y0.b0, y1.b0, 0, 0] | [0, 0, y2.b0, y3.b0]
      w0 = __builtin_amdgcn_perm(y[1], y[0], 0x0C0C0400u) | __builtin_amdgcn_perm(y[3], y[2], 0x04000C0Cu);
      w1 = __builtin_amdgcn_perm(y[5], y[4], 0x0C0C0400u) | __builtin_amdgcn_perm(y[7], y[6], 0x04000C0Cu);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w0 |= C::code(x[i], s) << (8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) w1 |= C::code(x[4 + i], s) << (8 * i);
    }
  }
  return make_uint2(w0, w1);
}

// Eight 4-bit codes of one lane, packed: code i in bits 4i .. 4i+3.
template <class C>
__device__ __forceinline__ uint32_t quantise8_nibbles(const float (&x)[8], float s) {
  uint32_t w = 0;
  if (s != 0.0f) {
    float q[8];
    quotients<8>(x, s, q);
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (code_bits(q[i], C::kQmax) & 0xFu) << (4 * i);
  }
  return w;
}

__device__ __forceinline__ void unpack8(uint4 raw, float (&x)[8], float& amax) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    amax = fmaxf(amax, fmaxf(fabsf(x[2 * i]), fabsf(x[2 * i + 1])));
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

}  // namespace kv8
