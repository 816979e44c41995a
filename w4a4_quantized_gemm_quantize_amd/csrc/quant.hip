// Activation / weight quantization kernels for gfx950.
//
// INT4 (APEX4, abstract: W4A4-g128 activations quantized per group of 128 along
// K; other group sizes for its mixed-granularity mode). Per group:
//   a = max|x|, s = fl32(a / 7), q = clamp(rne(fl32(x / s)), -8, 7), s = 0 and
//   q = 0 for an all-zero group. The rule only yields q in [-7, 7], stored
//   sign-magnitude: each 32-bit word holds the codes c0..c7 of 8 consecutive k;
//   byte b holds sign(c_b) in bit 7, |c_b| in bits 2..0, |c_(4+b)| in bits 6..4
//   and sign(c_(4+(b+3)%4)) in bit 3, the sign bit being that of the input value.
//   The GEMM turns a word into 8 FP8 E4M3 operand bytes with two masks and one
//   rotate.
// MXFP4 (the open-standard MXFP4 of the FP4 RL abstract; OCP MX v1.0 block
// rule): per 32 elements E = floor(log2 a) - 2, codes = E2M1(x / 2^E) with
// ties to even and saturation at 6, E8M0 byte E + 127. The scale bytes are
// written in 256-k panels (panel q = blocks 8q..8q+7 of every row, row after
// row, min(8, blocks left) bytes per row), so the GEMM reads one stage's scales
// of a tile as one contiguous run.
//
// Both kernels stream HBM: each lane loads 8 fp16 (one 128-bit load) per row
// it covers, a group's absmax is reduced across the lanes that hold it with DPP
// row permutes (no LDS), and each lane writes its 8 codes as one 32-bit store.
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

// 8 magnitudes (low bits of m[]) and the 8 fp16 inputs they came from -> one
// sign-magnitude word (layout in the file header).
__device__ __forceinline__ uint32_t pack8(const uint32_t m[8], uint4 raw) {
  const uint32_t p0 = (m[4] << 4) | m[0];     // byte 0 = |c0| | |c4| << 4
  const uint32_t p1 = (m[5] << 4) | m[1];
  const uint32_t p2 = (m[6] << 4) | m[2];
  const uint32_t p3 = (m[7] << 4) | m[3];
  const uint32_t lo = __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u);    // [p0.b0, p1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(p3, p2, 0x04000C0Cu);    // [0, 0, p2.b0, p3.b0]
  // high byte of each fp16 input: bit 7 = its sign
  const uint32_t s_lo = __builtin_amdgcn_perm(raw.y, raw.x, 0x07050301u);   // x0..x3
  const uint32_t s_hi = __builtin_amdgcn_perm(raw.w, raw.z, 0x07050301u);   // x4..x7
  const uint32_t s_hi_rot = __builtin_amdgcn_alignbit(s_hi, s_hi, 28);      // rotl 4: byte b bit 7 -> byte b+1 bit 3
  return (lo | hi) | (s_lo & 0x80808080u) | (s_hi_rot & 0x08080808u);
}

// Group scale and its reciprocal (r = 0 for an all-zero group so every code is 0).
__device__ __forceinline__ void group_scale(float a, float& s, float& r) {
  constexpr float r7 = 1.0f / 7.0f;      // RN(1/7), folded at compile time
  s = div_rn(a, 7.0f, r7);
  r = (s == 0.0f) ? 0.0f : 1.0f / s;     // correctly rounded division
}

__device__ __forceinline__ uint32_t int4_codes8(const float f[8], uint4 raw, float s, float r) {
  uint32_t m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = mag_code(div_rn(fabsf(f[i]), s, r));
  return pack8(m, raw);
}

// Lane mapping of the 2-D grid: a block is kQuantThreads lanes = (256 / W) row
// slots x W chunk columns, W in {64, 128, 256}; each lane covers kRowsPerThread
// rows spaced (256 / W) apart.
struct Map {
  int col;       // 8-element chunk index within the row
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

// One group of G elements spans G/8 consecutive lanes of one row.
template <int G>
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_groups(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int cpr, int wshift,
    uint32_t* __restrict__ q, float* __restrict__ s) {
  constexpr int LPG = G / 8;
  const Map mp = lane_map(wshift);
  if (mp.col >= cpr) return;                  // whole lane groups drop out together
  uint4 raw[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int row = mp.row0 + u * mp.rstep;
    if (row < M) raw[u] = *reinterpret_cast<const uint4*>(x + row * ldx + mp.col * 8);
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int row = mp.row0 + u * mp.rstep;
    if (row < M) {                            // uniform across each lane group
      float f[8];
      halves_to_float8(raw[u], f);
      float a = fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3])));
      a = fmaxf(a, fmaxf(fmaxf(fabsf(f[4]), fabsf(f[5])), fmaxf(fabsf(f[6]), fabsf(f[7]))));
      a = group_max<LPG>(a);
      float sc, rc;
      group_scale(a, sc, rc);
      q[(int64_t)row * cpr + mp.col] = int4_codes8(f, raw[u], sc, rc);
      if ((threadIdx.x & (LPG - 1)) == 0) s[(int64_t)(mp.col / LPG) * M + row] = sc;   // group-major
    }
  }
}

// Per-token quantization (one group spans the whole row): one block per row,
// absmax reduced across the block, then the row is read again from cache.
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_rows(
    const uint16_t* __restrict__ x, int64_t ldx, int cpr,
    uint32_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float wave_max[kQuantThreads / 64];
  const int row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  float a = 0.0f;
  for (int c = threadIdx.x; c < cpr; c += kQuantThreads) {
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
  float sc, rc;
  group_scale(a, sc, rc);
  for (int c = threadIdx.x; c < cpr; c += kQuantThreads) {
    const uint4 raw = *reinterpret_cast<const uint4*>(xr + c * 8);
    float f[8];
    halves_to_float8(raw, f);
    q[(int64_t)row * cpr + c] = int4_codes8(f, raw, sc, rc);
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
        // min(8, blocks left) bytes each
        const int b = mp.col >> 2, nb = cpr >> 2;
        const int pq = b >> 3, pw = min(8, nb - 8 * pq);
        e8m0[(int64_t)8 * rows * pq + (int64_t)row * pw + (b & 7)] = (uint8_t)(E + 127);
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
  uint32_t* qp = reinterpret_cast<uint32_t*>(q);
  const int cpr = (int)(K / 8);
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
