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
// Both kernels stream HBM: each lane loads 32 consecutive fp16 values of a row
// with 128-bit loads, an INT4 group's absmax is reduced across the lanes that
// hold it with DPP row permutes (no LDS; an MXFP4 block is one lane), and each
// lane writes its codes with one 16-byte store. The grid is 2-D (chunk run x
// row block), so no lane divides to find its row.
//
// Vector-ALU economy for the INT4 rule (the stream must not become ALU-bound;
// about 4 vector instructions per element):
//   * absmax: running max and min of the packed fp16 pairs with the three-input
//     packed max / min, then max(max, -min) -- one instruction per two values.
//   * x / s is computed as q0 = x*r, e = fma(-q0, s, x), q1 = fma(e, r, q0) with
//     r = RN(1/s) computed once per group; with r correctly rounded and q0 within
//     an ulp this Markstein-style correction yields RN(x/s) (P. Markstein, IBM
//     J. Res. Dev. 34(1), 1990). The GPU parity tests check it against the
//     oracle's IEEE divisions over every (absmax, x) pair of fp16 values. The
//     kernel runs it with r/8 and 8s in place of r and s (power-of-two factors,
//     so every step is the same rounding scaled by 1/8) and reads x straight from
//     its fp16 half (mixed-precision fma, no conversion): the result is t/8,
//     t = RN(x/s).
//   * s = RN(a/7) the same way with r7 = RN(1/7).
//   * rounding, clamp, sign and packing in one instruction: |t| <= 7 (1 + 2^-23),
//     so t/8 lies in the subnormal range of FP6 E2M3, spaced 1/8 apart, where
//     round-to-nearest-even to FP6 is rne(t) / 8 -- the field sign << 5 | |q|.
//     v_cvt_scalef32_2xpk16_fp6_f32 converts 32 such values (even k from its
//     first operand, odd k from its second) into the 192-bit stream of two
//     8-byte units, and an AND-OR per word folds it. The sign of t is that of x,
//     zero included: the correction is written as en = fma(q0, 8s, -x),
//     q1 = fma(-en, r/8, q0), whose zero results carry the sign of x.
#include <algorithm>

#include "device.h"
#include "launch.h"
#include "quant_common.h"

namespace w4a4 {

namespace {

constexpr int kQuantThreads = 256;
constexpr int64_t kMaxGridY = 65535;

typedef float v16f __attribute__((ext_vector_type(16)));

// Bits of a word at positions 3, 4 (mod 6), where the stream's first word is
// zero, and at 0, 5 (mod 6), where its third word is zero; together they cover
// every bit the second word can have set.
constexpr uint32_t kFoldX = 0x18618618u;
constexpr uint32_t kFoldY = 0x61861861u;

// Codes of the 2 NW fp16 values of w[0..NW) (NW = 16 or 8): the 192-bit FP6
// stream of up to 32 codes (int4_stream), folded into 8-byte units (out.x/y:
// codes 0..15, out.z/w: codes 16..31).
template <int NW>
__device__ __forceinline__ uint4 int4_codes(const uint32_t* w, float r8, float s8, float nz) {
  const v6u f = int4_stream<NW>(w, r8, s8, nz);
  return uint4{f[0] | (f[1] & kFoldX), f[2] | (f[1] & kFoldY),
               f[3] | (f[4] & kFoldX), f[5] | (f[4] & kFoldY)};
}

// Lane tile: a wave covers 64 / LPW rows x LPW consecutive 32-element chunks
// (LPW = max(G / 32, 4) lanes per row, the G/32 lanes of a group adjacent), the
// block's four waves consecutive chunk runs of the same rows; blockIdx.x walks
// along the rows (HBM is swept row block by row block). The lanes that store a
// group's scale hold consecutive rows of it, so the group-major scale array is
// written in runs of 64 / LPW rows (64 bytes at G <= 128) instead of lone
// 4-byte words. Row blocks beyond gridDim.y are taken in a loop.
// q16: the code array is 16-byte aligned (one store per lane).
template <int G>
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_groups(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int cpr, int q16,
    uint2* __restrict__ q, float* __restrict__ s) {
  constexpr int LPG = G / 32;
  constexpr int LPW = LPG > 4 ? LPG : 4;
  constexpr int RW = 64 / LPW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * (4 * LPW) + wave * LPW + (lane % LPW);
  if (col >= cpr) return;                      // whole groups drop out together
  const float nz = opaque_neg_zero();
  for (int rb = blockIdx.y; rb * RW < M; rb += gridDim.y) {
    const int row = rb * RW + lane / LPW;
    if (row >= M) break;                       // the last row block only
    uint4 raw[4];
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + col * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = src[j];
    uint32_t w[16];
    words16(raw, w);
    const float a = group_max<LPG>(absmax_words<16>(w));
    float sc, r8, s8;
    group_scale(a, sc, r8, s8);
    const uint4 c = int4_codes<16>(w, r8, s8, nz);
    const int64_t pair = (int64_t)row * cpr + col;     // 16-byte unit pair index
    if (q16) {
      reinterpret_cast<uint4*>(q)[pair] = c;
    } else {
      q[2 * pair] = uint2{c.x, c.y};
      q[2 * pair + 1] = uint2{c.z, c.w};
    }
    if (lane % LPG == 0) s[(int64_t)(col / LPG) * M + row] = sc;   // group-major
  }
}

// Per-token quantization (one group spans the whole row, K % 16 == 0): one
// block per row, absmax reduced across the block, then the row is read again
// from cache. Lanes take 32-element chunks; a 16-element tail goes to lane 0.
__global__ __launch_bounds__(kQuantThreads) void k_int4_quant_rows(
    const uint16_t* __restrict__ x, int64_t ldx, int K,
    uint2* __restrict__ q, float* __restrict__ s) {
  __shared__ float wave_max[kQuantThreads / 64];
  const int row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  const int n32 = K >> 5;
  const bool tail = (K & 16) != 0;
  float a = 0.0f;
  for (int c = threadIdx.x; c < n32; c += kQuantThreads) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + c * 32);
    uint4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = src[j];
    uint32_t w[16];
    words16(r, w);
    a = fmaxf(a, absmax_words<16>(w));
  }
  if (tail && threadIdx.x == 0) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + n32 * 32);
    const uint4 r0 = src[0], r1 = src[1];
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    a = fmaxf(a, absmax_words<8>(w));
  }
  a = group_max<64>(a);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) a = fmaxf(a, wave_max[w]);
  float sc, r8, s8;
  group_scale(a, sc, r8, s8);
  const float nz = opaque_neg_zero();
  uint2* qr = q + (int64_t)row * (K >> 4);
  for (int c = threadIdx.x; c < n32; c += kQuantThreads) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + c * 32);
    uint4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = src[j];
    uint32_t w[16];
    words16(r, w);
    const uint4 v = int4_codes<16>(w, r8, s8, nz);
    qr[2 * c] = uint2{v.x, v.y};
    qr[2 * c + 1] = uint2{v.z, v.w};
  }
  if (tail && threadIdx.x == 0) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + n32 * 32);
    const uint4 r0 = src[0], r1 = src[1];
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    const uint4 v = int4_codes<8>(w, r8, s8, nz);
    qr[2 * n32] = uint2{v.x, v.y};
  }
  if (threadIdx.x == 0) s[row] = sc;
}

// E2M1 codes of 32 fp16 values (16 words, even k in the low halves) divided by
// d = 2^E: v_cvt_scalef32_pk_fp4_f16 converts two fp16 values to the E2M1 codes
// of x / d, rounding to nearest of {0,0.5,1,1.5,2,3,4,6} with ties to even,
// saturating at 6 and keeping the sign of zero -- the OCP MX rule; the parity
// tests check it over every fp16 input. Byte i of output word j holds elements
// 8j + 2i (low nibble) and 8j + 2i + 1.
__device__ __forceinline__ uint4 e2m1_codes32(const uint32_t w[16], float d) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t v = 0;
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(v, __builtin_bit_cast(h2, w[4 * j]), d, 0);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(v, __builtin_bit_cast(h2, w[4 * j + 1]), d, 1);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(v, __builtin_bit_cast(h2, w[4 * j + 2]), d, 2);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(v, __builtin_bit_cast(h2, w[4 * j + 3]), d, 3);
    o[j] = v;
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

// Offset of the scale byte of (row, block b) in the panel layout of a matrix
// whose rows hold nbo blocks: panel b / 8, rows of pw = min(8, blocks left)
// bytes, the even blocks' bytes first.
__device__ __forceinline__ int64_t panel_offset(int rows, int nbo, int row, int b) {
  const int pq = b >> 3, pw = min(8, nbo - 8 * pq), j = b & 7;
  const int pos = (j & 1) ? ((pw + 1) >> 1) + (j >> 1) : (j >> 1);
  return (int64_t)8 * rows * pq + (int64_t)row * pw + pos;
}

// Output modes of the MXFP4 quantizer. APPEND_RESIDUAL and APPEND_COPY write a
// matrix twice as wide along K (2 nb blocks per row): block b and, at b + nb,
// the MX quantization of the residual x - deq(Q(x)) (the activation side of
// the appended-residual GEMM), or a copy of Q(x) (its weight side).
// APPEND_TIED is APPEND_RESIDUAL with the second scale tied to the first: the
// first pass takes the smallest E1 with max|x| <= 6 2^E1 (nothing clips), the
// second quantizes the residual at E2 = E1 - 2 (nothing clips either), which
// bounds the error by 2^(E1 + 3) / 64 per element.
enum { MX_PLAIN = 0, MX_APPEND_RESIDUAL = 1, MX_APPEND_COPY = 2, MX_APPEND_TIED = 3 };

// The E2M1 values (unit scale) of the 8 codes of a word, element 2i from the
// low nibble of byte i.
__device__ __forceinline__ void e2m1_values8(uint32_t w, float v[8]) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
}

// Block exponent E = floor(log2 a) - 2 of a block with absmax a (a is 0 or a
// normal fp32, so its biased exponent field is floor(log2 a) + 127), -127 for
// an all-zero block.
__device__ __forceinline__ int block_exponent(float a) {
  const int biased = (int)((__float_as_uint(a) >> 23) & 0xFF);
  return (a == 0.0f) ? -127 : biased - 127 - 2;
}

// Smallest E with a <= 6 2^E for a block with absmax a: with a = 2^e (1 + f),
// e - 2 when f <= 1/2 (4 (1 + f) <= 6), else e - 1; -125 for an all-zero block
// (2^-125 and 2^-127 are then the two scales, both normal in fp32).
__device__ __forceinline__ int block_exponent_noclip(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xFF) - 127;
  return (a == 0.0f) ? -125 : ((u & 0x7FFFFFu) <= 0x400000u ? e - 2 : e - 1);
}

// Lane tile: a lane takes one 32-element block of a row (absmax within the
// lane); a wave covers 8 rows x the 8 blocks of one 256-k panel, the block's
// four waves the next panels of the same rows, blockIdx.x walking along the
// rows. A wave's 64 scale bytes are then one contiguous run of the panel
// layout (8 rows x w_p bytes). Row blocks beyond gridDim.y are looped.
// q16: the code array is 16-byte aligned (one store per lane).
template <int MODE>
__global__ __launch_bounds__(kQuantThreads) void k_mxfp4_quant(
    const uint16_t* __restrict__ x, int64_t ldx, int rows, int nb, int q16,
    uint32_t* __restrict__ q, uint8_t* __restrict__ e8m0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = (blockIdx.x * 4 + wave) * 8 + (lane & 7);     // block of the row
  if (b >= nb) return;
  const int nbo = MODE == MX_PLAIN ? nb : 2 * nb;              // blocks per output row
  auto store_codes = [&](int row, int bo, uint4 c) {
    const int64_t unit = (int64_t)row * nbo + bo;             // 16-byte code unit
    if (q16) {
      reinterpret_cast<uint4*>(q)[unit] = c;
    } else {
      q[4 * unit] = c.x; q[4 * unit + 1] = c.y; q[4 * unit + 2] = c.z; q[4 * unit + 3] = c.w;
    }
  };
  for (int rb = blockIdx.y; rb * 8 < rows; rb += gridDim.y) {
    const int row = rb * 8 + (lane >> 3);
    if (row >= rows) break;                  // the last row block only
    uint4 raw[4];
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = src[i];
    uint32_t w[16];
    words16(raw, w);
    const float a = absmax_words<16>(w);
    const int E = MODE == MX_APPEND_TIED ? block_exponent_noclip(a) : block_exponent(a);
    const float d = (a == 0.0f && MODE != MX_APPEND_TIED) ? 1.0f
                                                          : __uint_as_float((uint32_t)(E + 127) << 23);   // 2^E, normal
    const uint4 c = e2m1_codes32(w, d);
    store_codes(row, b, c);
    e8m0[panel_offset(rows, nbo, row, b)] = (uint8_t)(E + 127);
    if constexpr (MODE == MX_APPEND_COPY) {
      store_codes(row, nb + b, c);
      e8m0[panel_offset(rows, nbo, row, nb + b)] = (uint8_t)(E + 127);
    } else if constexpr (MODE == MX_APPEND_RESIDUAL || MODE == MX_APPEND_TIED) {
      // r = x - deq(Q(x)), exact in fp32 (at most 16 significant bits); the
      // E2M1 value of each code comes back from the reverse conversion
      const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
      float r[32];
      float ar = 0.0f;
#pragma unroll
      for (int jw = 0; jw < 4; ++jw) {
        float v[8];
        e2m1_values8(cw[jw], v);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const int k = 8 * jw + i;
          const h2 xx = __builtin_bit_cast(h2, w[k >> 1]);
          r[k] = (float)xx.x - v[i] * d;
          r[k + 1] = (float)xx.y - v[i + 1] * d;
          ar = fmaxf(ar, fmaxf(fabsf(r[k]), fabsf(r[k + 1])));
        }
      }
      const int E2 = MODE == MX_APPEND_TIED ? E - 2 : block_exponent(ar);
#pragma unroll
      for (int k = 0; k < 32; ++k) r[k] = ldexpf(r[k], -E2);   // exact
      store_codes(row, nb + b, e2m1_codes32_f32(r));
      e8m0[panel_offset(rows, nbo, row, nb + b)] = (uint8_t)(E2 + 127);
    }
  }
}

}  // namespace

void launch_int4_quant(const void* x, int64_t M, int64_t K, int64_t ldx, int group,
                       uint8_t* q, float* s, hipStream_t stream) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint2* qp = reinterpret_cast<uint2*>(q);
  if (group != 64 && group != 128 && group != 256 && group != 512) {   // group == K (per token)
    hipLaunchKernelGGL(k_int4_quant_rows, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, xp, ldx, (int)K, qp, s);
    return;
  }
  const int cpr = (int)(K / 32);      // 32-element chunks per row (K % group == 0)
  const int m = (int)M;
  const int q16 = (reinterpret_cast<uintptr_t>(q) & 15) == 0;
  const int64_t rw = group >= 128 ? 2048 / group : 16;          // rows per wave, 64 / LPW
  const int64_t lpw = 64 / rw;
  const dim3 grid((unsigned)((cpr + 4 * lpw - 1) / (4 * lpw)),
                  (unsigned)std::min<int64_t>((M + rw - 1) / rw, kMaxGridY));
  switch (group) {
    case 64: hipLaunchKernelGGL(k_int4_quant_groups<64>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, q16, qp, s); return;
    case 128: hipLaunchKernelGGL(k_int4_quant_groups<128>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, q16, qp, s); return;
    case 256: hipLaunchKernelGGL(k_int4_quant_groups<256>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, q16, qp, s); return;
    default: hipLaunchKernelGGL(k_int4_quant_groups<512>, grid, dim3(kQuantThreads), 0, stream, xp, ldx, m, cpr, q16, qp, s); return;
  }
}

void launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ldx,
                        uint8_t* q, uint8_t* e8m0, int mode, hipStream_t stream) {
  const int nb = (int)(K / 32);
  const dim3 grid((unsigned)((nb + 31) / 32), (unsigned)std::min<int64_t>((rows + 7) / 8, kMaxGridY));
  const int q16 = (reinterpret_cast<uintptr_t>(q) & 15) == 0;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint32_t* qp = reinterpret_cast<uint32_t*>(q);
  switch (mode) {
    case MX_APPEND_RESIDUAL:
      hipLaunchKernelGGL(k_mxfp4_quant<MX_APPEND_RESIDUAL>, grid, dim3(kQuantThreads), 0, stream,
                         xp, ldx, (int)rows, nb, q16, qp, e8m0);
      return;
    case MX_APPEND_COPY:
      hipLaunchKernelGGL(k_mxfp4_quant<MX_APPEND_COPY>, grid, dim3(kQuantThreads), 0, stream,
                         xp, ldx, (int)rows, nb, q16, qp, e8m0);
      return;
    case MX_APPEND_TIED:
      hipLaunchKernelGGL(k_mxfp4_quant<MX_APPEND_TIED>, grid, dim3(kQuantThreads), 0, stream,
                         xp, ldx, (int)rows, nb, q16, qp, e8m0);
      return;
    default:
      hipLaunchKernelGGL(k_mxfp4_quant<MX_PLAIN>, grid, dim3(kQuantThreads), 0, stream,
                         xp, ldx, (int)rows, nb, q16, qp, e8m0);
      return;
  }
}

}  // namespace w4a4
