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

}  // namespace w4a4
