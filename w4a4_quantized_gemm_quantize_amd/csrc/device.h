// Device-side helpers shared by the gfx950 kernels of libw4a4.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace w4a4 {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// DPP-permuted copy of v (same-row lane exchange, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

constexpr int DPP_QUAD_1032 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;   // lane i <-> 15-i within a row of 16
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within each half row

// Max over aligned groups of LANES consecutive lanes (LANES in {2,4,8,16,32,64}).
// Every lane of a group must be active; the result is in every lane.
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  static_assert(LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32 || LANES == 64, "lanes");
  if constexpr (LANES >= 8) v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_QUAD_1032>(v));
  if constexpr (LANES >= 4) v = fmaxf(v, dpp<DPP_QUAD_2301>(v));
  if constexpr (LANES >= 16) v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  if constexpr (LANES >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (LANES >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Cache policy of the output stores: non-temporal. Y is written once and not
// read back by the kernel; the hint keeps it from displacing the operand slabs
// that later tiles re-read from L2 and the last-level cache.
constexpr int kStoreNT = 2;

// Raw buffer resource over [base, base + bytes): loads beyond the range read
// 0 and stores beyond it are dropped (the range check covers the vector
// offset). Word 3 is the CDNA raw-buffer format word (32-bit data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// A vector offset past any buffer resource of < 2^31 bytes: stores through it
// are dropped, even with a scalar offset < 2^31 added.
constexpr int kDroppedOffset = (int)0x80000000u;

}  // namespace w4a4
