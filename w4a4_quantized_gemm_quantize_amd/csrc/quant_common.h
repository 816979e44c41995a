// Device helpers shared by the quantizer kernels (INT4, MXFP4, NVFP4).
#pragma once

#include "device.h"

namespace w4a4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// max |x| over the 2 NW fp16 values of w[0..NW) (NW even), as fp32.
template <int NW>
__device__ __forceinline__ float absmax_words(const uint32_t* w) {
  h2 mx = {0, 0}, mn = {0, 0};
#pragma unroll
  for (int i = 0; i < NW; i += 2) {
    const h2 a = __builtin_bit_cast(h2, w[i]), b = __builtin_bit_cast(h2, w[i + 1]);
    mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, a), b);
    mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, a), b);
  }
  mx = __builtin_elementwise_maximum(mx, -mn);
  return fmaxf((float)mx.x, (float)mx.y);
}

// -0.0 held in a register: an fma with a literal -0 addend would be rewritten
// as a multiply, which cannot read an fp16 operand directly.
__device__ __forceinline__ float opaque_neg_zero() {
  float nz = -0.0f;
  asm volatile("" : "+v"(nz));
  return nz;
}

// The 16 words of four 16-byte loads, in memory order.
__device__ __forceinline__ void words16(const uint4 r[4], uint32_t w[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[4 * j] = r[j].x; w[4 * j + 1] = r[j].y; w[4 * j + 2] = r[j].z; w[4 * j + 3] = r[j].w;
  }
}

// E2M1 codes of 32 fp32 values already divided by their block scale, two per
// instruction with unit scale: v_cvt_scalef32_pk_fp4_f32 rounds to the nearest
// of {0, 0.5, 1, 1.5, 2, 3, 4, 6} with ties to the even code, saturates at 6
// and keeps the sign of zero. Byte i of output word j holds elements 8j + 2i
// (low nibble) and 8j + 2i + 1.
__device__ __forceinline__ uint4 e2m1_codes32_f32(const float v[32]) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j], v[8 * j + 1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j + 2], v[8 * j + 3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j + 4], v[8 * j + 5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * j + 6], v[8 * j + 7], 1.0f, 3);
    o[j] = w;
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

// ---- INT4 rule (symmetric, s = fl32(a / 7), q = rne(fl32(x / s))): shared by
// the quantizer and the GEMM kernels that quantize their own activations, so
// both take every decision with the same instructions.

typedef float v16f_q __attribute__((ext_vector_type(16)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));

// Correctly rounded x / d given r = RN(1/d) (d normal, no overflow/underflow).
__device__ __forceinline__ float div_rn(float x, float d, float r) {
  const float q0 = x * r;
  const float e = fmaf(-q0, d, x);
  return fmaf(e, r, q0);
}

// Group scale s, and r8 = RN(1/s) / 8, s8 = 8 s for the scaled division
// (r8 = 0 for an all-zero group, so every code is a zero of the input's sign).
__device__ __forceinline__ void group_scale(float a, float& s, float& r8, float& s8) {
  constexpr float r7 = 1.0f / 7.0f;      // RN(1/7), folded at compile time
  s = div_rn(a, 7.0f, r7);
  r8 = ((s == 0.0f) ? 0.0f : 1.0f / s) * 0.125f;   // correctly rounded division
  s8 = s * 8.0f;
}

// t / 8 with t = RN(x / s), sign of x kept on zero results. nz is -0.0 held in a
// register (an fma with a literal -0 addend would be rewritten as a multiply,
// which cannot read the fp16 operand directly).
__device__ __forceinline__ float quot8(_Float16 h, float r8, float s8, float nz) {
  const float x = (float)h;
  const float q0 = fmaf(x, r8, nz);
  const float en = fmaf(q0, s8, -x);
  return fmaf(-en, r8, q0);
}

// The 192-bit FP6 E2M3 stream of the codes of the 2 NW fp16 values of
// w[0..NW) (NW = 16 or 8; missing values are zero codes): field k (bits 6k ..
// 6k+5) is sign << 5 | |q_k|, the operand form of the block-scaled FP6 matrix
// instruction. v_cvt_scalef32_2xpk16_fp6_f32 rounds t/8 (|t| <= 7 (1 + 2^-23),
// the subnormal range of FP6 E2M3, spaced 1/8) to nearest even: rne(t) / 8.
template <int NW>
__device__ __forceinline__ v6u int4_stream(const uint32_t* w, float r8, float s8, float nz) {
  v16f_q ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < NW) {
      const h2 v = __builtin_bit_cast(h2, w[i]);
      ev[i] = quot8(v.x, r8, s8, nz);   // k = 2i   -> field 2i
      od[i] = quot8(v.y, r8, s8, nz);   // k = 2i+1 -> field 2i+1
    } else {
      ev[i] = 0.0f;
      od[i] = 0.0f;
    }
  }
  const auto f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
  return v6u{f[0], f[1], f[2], f[3], f[4], f[5]};
}

}  // namespace w4a4
