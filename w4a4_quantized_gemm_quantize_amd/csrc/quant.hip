// Activation / weight quantization kernels for gfx950.
//
// INT4 (APEX4, abstract: W4A4-g128 activations quantized per group of 128 along
// K; other group sizes for its mixed-granularity mode). Per group:
//   a = max|x|, s = fl32(a / 7), q = clamp(rne(fl32(x / s)), -8, 7), s = 0 and
//   q = 0 for an all-zero group. The rule only yields q in [-7, 7], stored
//   sign-magnitude in 4 bits per code, the sign bit being that of the input
//   value: each 8-byte unit holds the codes c0..c15 of 16 consecutive k as two
//   32-bit words X, Y folded from the 96-bit stream S of the 6-bit fields
//   f_k = sign << 5 | |c_k| at bits 6k (the FP6 E2M3 encoding of the subnormal
//   +-|c_k|/8): X = S0 | (S1 & kFoldX), Y = S2 | (S1 & kFoldY). The GEMM
//   rebuilds S0, S1, S2 -- its FP6 operand -- with two ANDs and an AND-OR.
// MXFP4 (the open-standard MXFP4 of the FP4 RL abstract; OCP MX v1.0 block
// rule): per 32 elements E = floor(log2 a) - 2, codes = E2M1(x / 2^E) with
// ties to even and saturation at 6, E8M0 byte E + 127. The scale bytes are
// written in 256-k panels (panel q = blocks 8q..8q+7 of every row, row after
// row, min(8, blocks left) bytes per row, the even blocks' bytes first), so the
// GEMM reads one stage's scales of a tile as one contiguous run and a lane's
// bytes as one dword.
//
// Both kernels stream HBM: each lane loads 16 (INT4) or 8 (MXFP4) fp16 values
// per row it covers with 128-bit loads, a group's absmax is reduced across the
// lanes that hold it with DPP row permutes (no LDS), and each lane writes its
// codes with one store (64-bit INT4 word, 32-bit E2M1 word).
// The grid is 2-D (chunk column x row block), so no lane divides to find its row.
//
// Vector-ALU economy for the INT4 rule (the stream must not become ALU-bound):
//   * x / s is computed as q0 = x*r, e = fma(-q0, s, x), q1 = fma(e, r, q0) with
//     r = RN(1/s) computed once per group; with r correctly rounded and q0 within
//     an ulp this Markstein-style correction yields RN(x/s) (P. Markstein, IBM
//     J. Res. Dev. 34(1), 1990). The GPU parity tests check it against the
//     oracle's IEEE divisions over every (absmax, x) pair of fp16 values.
//   * s = RN(a/7) the same way with r7 = RN(1/7).
//   * rne + clamp on the magnitude: RNE is symmetric, so |q| = rne(|x| / s);
//     t = |x|/s is clamped to [0, 7] and 2^23 is added (binary32 spacing is 1 on
//     [2^23, 2^24), so the add rounds half-to-even) leaving |q| in the low bits.
#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kRowsPerThread = 4;   // independent 16-byte loads in flight per lane
constexpr float kMagic = 8388608.0f;    // 2^23

// Correctly rounded x / d given r = RN(1/d) (d normal, no overflow/underflow).
__device__ __forceinline__ float div_rn(float x, float d, float r) {
  const float q0 = x * r;
  const float e = fmaf(-q0, d, x);
  return fmaf(e, r, q0);
}

// |q| = min(rne(t), 7) for t >= 0, in the low 3 bits of the returned word.
__device__ __forceinline__ uint32_t mag_code(float t) {
  return __float_as_uint(__builtin_amdgcn_fmed3f(t, 0.0f, 7.0f) + kMagic);
}

// Bits of a word at positions 3, 4 (mod 6), where the stream's first word is
// zero, and at 0, 5 (mod 6), where its third word is zero; together they cover
// every bit the second word can have set.
constexpr uint32_t kFoldX = 0x18618618u;
constexpr uint32_t kFoldY = 0x61861861u;

// 16 magnitudes (low 3 bits of m[]) and the 16 fp16 inputs they came from
// (r0: inputs 0..7, r1: 8..15) -> the 8-byte INT4 unit (layout in the header).
__device__ __forceinline__ uint2 pack16(const uint32_t m[16], uint4 r0, uint4 r1) {
  const uint32_t h[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  uint32_t f[16];
#pragma unroll
  for (int k = 0; k < 16; ++k)    // FP6 field: sign of input k (fp16 bit 15) << 5 | |c_k|
    f[k] = (m[k] & 7u) | (((h[k >> 1] >> (16 * (k & 1) + 15)) & 1u) << 5);
  const uint32_t s0 = f[0] | f[1] << 6 | f[2] << 12 | f[3] << 18 | f[4] << 24 | f[5] << 30;
  const uint32_t s1 = f[5] >> 2 | f[6] << 4 | f[7] << 10 | f[8] << 16 | f[9] << 22 | f[10] << 28;
  const uint32_t s2 = f[10] >> 4 | f[11] << 2 | f[12] << 8 | f[13] << 14 | f[14] << 20 | f[15] << 26;
  return uint2{s0 | (s1 & kFoldX), s2 | (s1 & kFoldY)};
}

// Group scale and its reciprocal (r = 0 for an all-zero group so every code is 0).
__device__ __forceinline__ void group_scale(float a, float& s, float& r) {
  constexpr float r7 = 1.0f / 7.0f;      // RN(1/7), folded at compile time
  s = div_rn(a, 7.0f, r7);
  r = (s == 0.0f) ? 0.0f : 1.0f / s;     // correctly rounded division
}

__device__ __forceinline__ uint2 int4_codes16(const float f[16], uint4 r0, uint4 r1, float s, float r) {
  uint32_t m[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) m[i] = mag_code(div_rn(fabsf(f[i]), s, r));
  return pack16(m, r0, r1);
}

// Lane mapping of the 2-D grid: a block is kQuantThreads lanes = (256 / W) row
// slots x W chunk columns, W in {64, 128, 256}; each lane covers kRowsPerThread
// rows spaced (256 / W) apart.
struct Map {
  int col;       // chunk index within the row (16 elements INT4, 8 MXFP4)
  int row0;      // first row
  int rstep;     // row spacing between a lane's rows
};

__device__ __forceinline__ Map lane_map(int wshift) {
  const int W = 1 << wshift;
  Map m;
  m.col = blockIdx.x * W + (threadIdx.x & (W - 1));
  m.rstep = kQuantThreads >> wshift;
  m.row0 = blockIdx.y * m.rstep * kRowsPerThread + (threadIdx.x >> wshift);
  return m;
}

// One group of G elements spans G/16 consecutive lanes of one row; a lane
// covers 16 elements (chunk col) of each of its rows.
template <int G>
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_groups(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int cpr, int wshift,
    uint2* __restrict__ q, float* __restrict__ s) {
  constexpr int LPG = G / 16;
  const Map mp = lane_map(wshift);
  if (mp.col >= cpr) return;                  // whole lane groups drop out together
  uint4 raw[kRowsPerThread][2];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int row = mp.row0 + u * mp.rstep;
    if (row < M) {
      const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + mp.col * 16);
      raw[u][0] = src[0];
      raw[u][1] = src[1];
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int row = mp.row0 + u * mp.rstep;
    if (row < M) {                            // uniform across each lane group
      float f[16];
      halves_to_float8(raw[u][0], f);
      halves_to_float8(raw[u][1], f + 8);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(f[i]));
      a = group_max<LPG>(a);
      float sc, rc;
      group_scale(a, sc, rc);
      q[(int64_t)row * cpr + mp.col] = int4_codes16(f, raw[u][0], raw[u][1], sc, rc);
      if ((threadIdx.x & (LPG - 1)) == 0) s[(int64_t)(mp.col / LPG) * M + row] = sc;   // group-major
    }
  }
}

// Per-token quantization (one group spans the whole row): one block per row,
// absmax reduced across the block, then the row is read again from cache.
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_rows(
    const uint16_t* __restrict__ x, int64_t ldx, int cpr,
    uint2* __restrict__ q, float* __restrict__ s) {
  __shared__ float wave_max[kQuantThreads / 64];
  const int row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  float a = 0.0f;
  for (int c = threadIdx.x; c < cpr; c += kQuantThreads) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + c * 16);
    float f[16];
    halves_to_float8(src[0], f);
    halves_to_float8(src[1], f + 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(f[i]));
  }
  a = group_max<64>(a);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) a = fmaxf(a, wave_max[w]);
  float sc, rc;
  group_scale(a, sc, rc);
  for (int c = threadIdx.x; c < cpr; c += kQuantThreads) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + c * 16);
    const uint4 r0 = src[0], r1 = src[1];
    float f[16];
    halves_to_float8(r0, f);
    halves_to_float8(r1, f + 8);
    q[(int64_t)row * cpr + c] = int4_codes16(f, r0, r1, sc, rc);
  }
  if (threadIdx.x == 0) s[row] = sc;
}

// E2M1 conversion of 8 values already divided by 2^E, two per instruction:
// v_cvt_scalef32_pk_fp4_f32 (unit scale) rounds to nearest of
// {0,0.5,1,1.5,2,3,4,6}, ties to even, saturates at 6 and keeps the sign of
// zero -- the OCP MX rule; the parity tests check it over every fp16 input.
__device__ __forceinline__ uint32_t e2m1_codes8(const float v[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// 32-element block = 4 lanes x 8 values.
__global__ __launch_bounds__(kQuantThreads) void k_mxfp4_quant(
    const uint16_t* __restrict__ x, int64_t ldx, int rows, int cpr, int wshift,
    uint32_t* __restrict__ q, uint8_t* __restrict__ e8m0) {
  const Map mp = lane_map(wshift);
  if (mp.col >= cpr) return;
  uint4 raw[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int row = mp.row0 + u * mp.rstep;
    if (row < rows) raw[u] = *reinterpret_cast<const uint4*>(x + row * ldx + mp.col * 8);
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int row = mp.row0 + u * mp.rstep;
    if (row < rows) {
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
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ldexpf(f[i], -E);   // exact power-of-two scaling
      q[(int64_t)row * cpr + mp.col] = e2m1_codes8(v);
      if ((threadIdx.x & 3) == 0) {
        // panel layout: block b of the row goes to panel b / 8, whose rows hold
        // pw = min(8, blocks left) bytes each, the even blocks' bytes first
        const int b = mp.col >> 2, nb = cpr >> 2;
        const int pq = b >> 3, pw = min(8, nb - 8 * pq), j = b & 7;
        const int pos = (j & 1) ? ((pw + 1) >> 1) + (j >> 1) : (j >> 1);
        e8m0[(int64_t)8 * rows * pq + (int64_t)row * pw + pos] = (uint8_t)(E + 127);
      }
    }
  }
}

int width_shift(int cpr) { return cpr <= 64 ? 6 : cpr <= 128 ? 7 : 8; }

dim3 grid_for(int rows, int cpr, int wshift) {
  const int W = 1 << wshift;
  const int rows_per_block = (kQuantThreads >> wshift) * kRowsPerThread;
  return dim3((unsigned)((cpr + W - 1) / W), (unsigned)((rows + rows_per_block - 1) / rows_per_block));
}

}  // namespace

void launch_int4_quant(const void* x, int64_t M, int64_t K, int64_t ldx, int group,
                       uint8_t* q, float* s, hipStream_t stream) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint2* qp = reinterpret_cast<uint2*>(q);
  const int cpr = (int)(K / 16);      // 16-element chunks per row
  const int ws = width_shift(cpr);
  const dim3 grid = grid_for((int)M, cpr, ws);
  const int m = (int)M;
  switch (group == K && group > 512 ? 0 : group) {
    case 64: hipLaunchKernelGGL(k_int4_quant_groups<64>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, ws, qp, s); return;
    case 128: hipLaunchKernelGGL(k_int4_quant_groups<128>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, ws, qp, s); return;
    case 256: hipLaunchKernelGGL(k_int4_quant_groups<256>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, ws, qp, s); return;
    case 512: hipLaunchKernelGGL(k_int4_quant_groups<512>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, ws, qp, s); return;
    default:  // group == K (per token), validated by the caller
      hipLaunchKernelGGL(k_int4_quant_rows, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, xp, ldx, cpr, qp, s);
      return;
  }
}

void launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ldx,
                        uint8_t* q, uint8_t* e8m0, hipStream_t stream) {
  const int cpr = (int)(K / 8);
  const int ws = width_shift(cpr);
  hipLaunchKernelGGL(k_mxfp4_quant, grid_for((int)rows, cpr, ws), dim3(kQuantThreads), 0, stream,
                     static_cast<const uint16_t*>(x), ldx, (int)rows, cpr, ws,
                     reinterpret_cast<uint32_t*>(q), e8m0);
}

}  // namespace w4a4
