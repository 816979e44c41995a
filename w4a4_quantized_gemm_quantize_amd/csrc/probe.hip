// On-chip peak probes for gfx950: the rates a kernel on this GPU can reach,
// measured rather than taken from a data sheet, so a roofline fraction can be
// stated against both. Not part of the W4A4 computation.
//
//  * matrix-core loops: every wave issues back-to-back MFMAs of one kind into
//    four independent accumulators (no dependency stalls), on operand bits
//    drawn from a per-lane hash (the matrix cores' power draw, hence their
//    clock, depends on the data: all-zero operands run faster than the codes
//    of a real GEMM);
//  * HBM streams: a grid-stride read of a buffer (16-byte loads, XOR-folded so
//    nothing is optimized away), and a copy of one buffer into another.
#include "device.h"

namespace w4a4 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Operand words of this lane: pseudo-random bits. FP8 / FP6 / FP4 patterns
// that encode NaN or infinity are avoided by clearing each byte's top
// exponent bit (FP8 E4M3 0x7F / 0xFF are the only NaNs; FP6 and FP4 have none);
// fp16 words keep their exponent below 31 the same way.
__device__ __forceinline__ uint32_t operand_word(int i) {
  const uint32_t h = mix((uint32_t)(blockIdx.x * blockDim.x + threadIdx.x) * 16u + (uint32_t)i + 1u);
  return h & 0xBFBFBFBFu;
}

enum { P_INT8 = 0, P_FP8 = 1, P_FP6 = 2, P_FP4 = 3, P_FP16 = 4, P_VALU_F32 = 5 };

template <int KIND>
__global__ __launch_bounds__(256) void k_probe_mfma(int64_t iters, float* __restrict__ sink) {
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)operand_word(i);
    b[i] = (int)operand_word(8 + i);
  }
  float out = 0.0f;
  if constexpr (KIND == P_VALU_F32) {
    // 16 independent fp32 fma chains per lane, 4 steps each per iteration
    // (64 v_fma_f32 per iteration, the same count as the MFMA loops' 4 per
    // iteration times 16), scalar fp32: the vector unit's non-packed rate
    float f[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = __uint_as_float((operand_word(i) & 0x007FFFFFu) | 0x3F800000u);
    const float m = __uint_as_float(0x3F7FFFF0u), c = 1.0e-7f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = fmaf(f[i], m, c);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) out += f[i];
  } else if constexpr (KIND == P_INT8) {
    const v4i a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b4, a4, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b4, b4, c3, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) out += (float)(c0[r] ^ c1[r] ^ c2[r] ^ c3[r]);
  } else if constexpr (KIND == P_FP16) {
    const v8h a8 = __builtin_bit_cast(v8h, v4i{a[0], a[1], a[2], a[3]});
    const v8h b8 = __builtin_bit_cast(v8h, v4i{b[0], b[1], b[2], b[3]});
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, b8, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b8, a8, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, a8, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b8, b8, c3, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) out += c0[r] + c1[r] + c2[r] + c3[r];
  } else {
    // block-scaled f8f6f4: format code 0 = FP8 E4M3, 2 = FP6 E2M3, 4 = FP4 E2M1
    constexpr int F = KIND == P_FP8 ? 0 : KIND == P_FP6 ? 2 : 4;
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, F, F, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, F, F, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, F, F, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, F, F, 0, 127, 0, 127);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) out += c0[r] + c1[r] + c2[r] + c3[r];
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = out;
}

// XOR of every 16-byte word of buf (n16 words), one partial per thread.
__global__ __launch_bounds__(256) void k_probe_read(const uint4* __restrict__ buf, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = buf[i], v1 = buf[i + stride], v2 = buf[i + 2 * stride], v3 = buf[i + 3 * stride];
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^
           v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_probe_copy(const uint4* __restrict__ src, int64_t n16,
                                                   uint4* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

// Launch shapes of the probes: MFMA loops run 4 waves per workgroup, 8
// workgroups per CU (two waves per SIMD twice over); streams 4 workgroups of
// 256 threads per CU, grid-stride.
constexpr int kProbeMfmaBlocks = 256 * 8;
constexpr int kProbeStreamBlocks = 256 * 4;

int64_t probe_mfma_sink_floats() { return (int64_t)kProbeMfmaBlocks * 256; }
int64_t probe_stream_sink_words() { return (int64_t)kProbeStreamBlocks * 256; }

int64_t probe_mfma_ops(int kind) {
  switch (kind) {
    case P_INT8: return 2LL * 32 * 32 * 32;
    case P_FP16: return 2LL * 32 * 32 * 16;
    case P_FP8: case P_FP6: case P_FP4: return 2LL * 32 * 32 * 64;
    case P_VALU_F32: return 2LL * 64 * 16;   // a lane's 64 fmas of one iteration = 4 x 16 (4 "instructions" per iteration below)
    default: return 0;
  }
}

void launch_probe_mfma(int kind, int64_t iters, float* sink, hipStream_t stream) {
  const dim3 grid(kProbeMfmaBlocks), block(256);
  switch (kind) {
    case P_INT8: hipLaunchKernelGGL((k_probe_mfma<P_INT8>), grid, block, 0, stream, iters, sink); break;
    case P_FP8: hipLaunchKernelGGL((k_probe_mfma<P_FP8>), grid, block, 0, stream, iters, sink); break;
    case P_FP6: hipLaunchKernelGGL((k_probe_mfma<P_FP6>), grid, block, 0, stream, iters, sink); break;
    case P_FP4: hipLaunchKernelGGL((k_probe_mfma<P_FP4>), grid, block, 0, stream, iters, sink); break;
    case P_VALU_F32: hipLaunchKernelGGL((k_probe_mfma<P_VALU_F32>), grid, block, 0, stream, iters, sink); break;
    default: hipLaunchKernelGGL((k_probe_mfma<P_FP16>), grid, block, 0, stream, iters, sink); break;
  }
}

void launch_probe_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_probe_read, dim3(kProbeStreamBlocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
}

void launch_probe_copy(const void* src, int64_t bytes, void* dst, hipStream_t stream) {
  hipLaunchKernelGGL(k_probe_copy, dim3(kProbeStreamBlocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, static_cast<uint4*>(dst));
}

}  // namespace w4a4

// ------------------------------------------------------------------ C ABI
#include "w4a4_probe.h"

extern "C" {

int64_t w4a4_probe_sink_bytes(void) {
  const int64_t a = w4a4::probe_mfma_sink_floats() * 4, b = w4a4::probe_stream_sink_words() * 4;
  return a > b ? a : b;
}

int64_t w4a4_probe_mfma_ops(int32_t kind, int64_t iters) {
  const int64_t per = w4a4::probe_mfma_ops(kind);
  if (per == 0 || iters < 0) return -1;
  // 4 waves per workgroup, 4 MFMAs per iteration
  return per * 4 * iters * 4 * (int64_t)w4a4::kProbeMfmaBlocks;
}

w4a4_status_t w4a4_probe_mfma(int32_t kind, int64_t iters, void* sink, void* stream) {
  if (kind < W4A4_PROBE_INT8 || kind > W4A4_PROBE_VALU_F32 || iters <= 0) return W4A4_E_SHAPE;
  if (!sink) return W4A4_E_NULL;
  if (reinterpret_cast<uintptr_t>(sink) % 4) return W4A4_E_ALIGN;
  w4a4::launch_probe_mfma(kind, iters, static_cast<float*>(sink), static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? W4A4_OK : W4A4_E_HIP;
}

w4a4_status_t w4a4_probe_hbm_read(const void* buf, int64_t bytes, void* sink, void* stream) {
  if (bytes <= 0 || bytes % 16) return W4A4_E_SHAPE;
  if (!buf || !sink) return W4A4_E_NULL;
  if (reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(sink) % 4) return W4A4_E_ALIGN;
  w4a4::launch_probe_read(buf, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? W4A4_OK : W4A4_E_HIP;
}

w4a4_status_t w4a4_probe_hbm_copy(const void* src, int64_t bytes, void* dst, void* stream) {
  if (bytes <= 0 || bytes % 16) return W4A4_E_SHAPE;
  if (!src || !dst) return W4A4_E_NULL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return W4A4_E_ALIGN;
  w4a4::launch_probe_copy(src, bytes, dst, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? W4A4_OK : W4A4_E_HIP;
}

}  // extern "C"
