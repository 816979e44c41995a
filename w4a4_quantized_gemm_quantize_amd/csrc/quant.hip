// Activation / weight quantization kernels for gfx950.
//
// INT4 (APEX4, abstract: W4A4-g128 activations quantized per group of 128 along
// K; other group sizes for its mixed-granularity mode). Per group:
//   a = max|x|, s = fl32(a / 7), q = clamp(rne(fl32(x / s)), -8, 7), s = 0 and
//   q = 0 for an all-zero group; two codes per byte, even k in the low nibble.
// MXFP4 (the open-standard MXFP4 of the FP4 RL abstract; OCP MX v1.0 block
// rule): per 32 elements E = floor(log2 a) - 2, codes = E2M1(x / 2^E) with
// ties to even and saturation at 6, E8M0 byte E + 127.
//
// Both kernels are HBM-bound streams: each lane loads 8 fp16 (one 128-bit load),
// a group's absmax is reduced across the lanes that hold it with DPP row
// permutes (no LDS), and each lane writes its 8 codes as one 32-bit store.
#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kChunksPerThread = 4;  // independent 16-byte loads in flight per lane

// Quantize 8 values with scale s (s > 0) or to zero (s == 0); pack 8 nibbles.
__device__ __forceinline__ uint32_t int4_codes8(const float f[8], float s) {
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float t = f[i] / s;                       // correctly rounded binary32 division
    float r = fminf(fmaxf(rintf(t), -8.0f), 7.0f);
    int q = (s == 0.0f) ? 0 : (int)r;
    word |= (uint32_t)(q & 0xF) << (4 * i);
  }
  return word;
}

// One group of G elements spans G/8 consecutive lanes.
template <int G>
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_groups(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t M, int64_t K,
    uint32_t* __restrict__ q, float* __restrict__ s) {
  constexpr int LPG = G / 8;
  const int64_t cpr = K / 8;                  // 8-element chunks per row
  const int64_t total = M * cpr;
  const int64_t base = (int64_t)blockIdx.x * (kQuantThreads * kChunksPerThread) + threadIdx.x;
  uint4 raw[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int64_t c = base + u * kQuantThreads;
    if (c < total) {
      const int64_t row = c / cpr, col = c - row * cpr;
      raw[u] = *reinterpret_cast<const uint4*>(x + row * ldx + col * 8);
    }
  }
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int64_t c = base + u * kQuantThreads;
    if (c < total) {                          // uniform across each lane group
      float f[8];
      halves_to_float8(raw[u], f);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
      a = group_max<LPG>(a);
      const float sc = a / 7.0f;
      const int64_t row = c / cpr, col = c - row * cpr;
      q[row * (K / 8) + col] = int4_codes8(f, sc);
      if ((threadIdx.x & (LPG - 1)) == 0) s[row * (K / G) + (col * 8) / G] = sc;
    }
  }
}

// Per-token quantization (one group spans the whole row): one block per row,
// absmax reduced across the block, then the row is read again from cache.
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_rows(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t K,
    uint32_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float wave_max[kQuantThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  const int64_t cpr = K / 8;
  float a = 0.0f;
  for (int64_t c = threadIdx.x; c < cpr; c += kQuantThreads) {
    float f[8];
    halves_to_float8(*reinterpret_cast<const uint4*>(xr + c * 8), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  }
  a = group_max<64>(a);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) a = fmaxf(a, wave_max[w]);
  const float sc = a / 7.0f;
  for (int64_t c = threadIdx.x; c < cpr; c += kQuantThreads) {
    float f[8];
    halves_to_float8(*reinterpret_cast<const uint4*>(xr + c * 8), f);
    q[row * cpr + c] = int4_codes8(f, sc);
  }
  if (threadIdx.x == 0) s[row] = sc;
}

// Round |v| (already divided by 2^E) to an E2M1 magnitude index 0..7:
// nearest of {0,0.5,1,1.5,2,3,4,6}, ties to the even index, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_index(float m) {
  uint32_t i = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) +
               (m > 2.5f) + (m >= 3.5f) + (m > 5.0f);
  return i;
}

// 32-element block = 4 lanes x 8 values.
__global__ __launch_bounds__(kQuantThreads) void k_mxfp4_quant(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t rows, int64_t K,
    uint32_t* __restrict__ q, uint8_t* __restrict__ e8m0) {
  const int64_t cpr = K / 8;
  const int64_t total = rows * cpr;
  const int64_t base = (int64_t)blockIdx.x * (kQuantThreads * kChunksPerThread) + threadIdx.x;
  uint4 raw[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int64_t c = base + u * kQuantThreads;
    if (c < total) {
      const int64_t row = c / cpr, col = c - row * cpr;
      raw[u] = *reinterpret_cast<const uint4*>(x + row * ldx + col * 8);
    }
  }
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int64_t c = base + u * kQuantThreads;
    if (c < total) {
      float f[8];
      halves_to_float8(raw[u], f);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
      a = group_max<4>(a);
      // a is 0 or a normal fp32 (fp16 values widen to normal fp32), so its
      // biased exponent field is floor(log2 a) + 127.
      const int biased = (int)((__float_as_uint(a) >> 23) & 0xFF);
      const int E = (a == 0.0f) ? -127 : biased - 127 - 2;
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = ldexpf(f[i], -E);      // exact power-of-two scaling
        const uint32_t sign = (__float_as_uint(f[i]) >> 31) & 1u;
        word |= ((sign << 3) | e2m1_index(fabsf(v))) << (4 * i);
      }
      const int64_t row = c / cpr, col = c - row * cpr;
      q[row * cpr + col] = word;
      if ((threadIdx.x & 3) == 0) e8m0[row * (K / 32) + col / 4] = (uint8_t)(E + 127);
    }
  }
}

}  // namespace

void launch_int4_quant(const void* x, int64_t M, int64_t K, int64_t ldx, int group,
                       uint8_t* q, float* s, hipStream_t stream) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint32_t* qp = reinterpret_cast<uint32_t*>(q);
  const int64_t total = M * (K / 8);
  const int64_t per_block = kQuantThreads * kChunksPerThread;
  const dim3 grid((unsigned)((total + per_block - 1) / per_block));
  switch (group) {
    case 64: hipLaunchKernelGGL(k_int4_quant_groups<64>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, M, K, qp, s); return;
    case 128: hipLaunchKernelGGL(k_int4_quant_groups<128>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, M, K, qp, s); return;
    case 256: hipLaunchKernelGGL(k_int4_quant_groups<256>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, M, K, qp, s); return;
    case 512: hipLaunchKernelGGL(k_int4_quant_groups<512>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, M, K, qp, s); return;
    default:  // group == K, validated by the caller
      hipLaunchKernelGGL(k_int4_quant_rows, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, xp, ldx, K, qp, s);
      return;
  }
}

void launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ldx,
                        uint8_t* q, uint8_t* e8m0, hipStream_t stream) {
  const int64_t total = rows * (K / 8);
  const int64_t per_block = kQuantThreads * kChunksPerThread;
  const dim3 grid((unsigned)((total + per_block - 1) / per_block));
  hipLaunchKernelGGL(k_mxfp4_quant, grid, dim3(kQuantThreads), 0, stream,
                     static_cast<const uint16_t*>(x), ldx, rows, K, reinterpret_cast<uint32_t*>(q), e8m0);
}

}  // namespace w4a4
