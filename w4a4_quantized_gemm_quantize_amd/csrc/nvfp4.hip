// NVFP4 for gfx950: global scale, quantizer and GEMM.
//
// NVFP4 (ARCQuant abstract, APEX4 page: the fine-grained FP4 format a standard
// GEMM consumes; Minima abstract, "Daily Papers" page: 16-element block
// scaling plus a calibrated global scale per module): FP4 E2M1 elements in
// blocks of 16 along K, each block with an FP8 E4M3 scale s_b, the tensor with
// one binary32 global scale s_g, x_hat = v * s_b * s_g. Per block with absmax a:
//   d = fl32(6 s_g); s_b = E4M3(min(fl32(a / d), 448)), s_b = 0 when a = 0;
//   e = fl32(1 / fl32(s_b s_g)), e = 0 when that product is 0;
//   code = E2M1(fl32(x e)), nearest with ties to the even code, saturating at
//   6, the sign bit that of x.
// Every binary32 step is correctly rounded (the divisions are IEEE divisions,
// one per block); v_cvt_pk_fp8_f32 rounds to nearest even into OCP E4M3 with
// subnormals, and v_cvt_scalef32_pk_fp4_f32 with unit scale does the E2M1
// rounding. The default global scale is fl32(max|x| / 2688), 2688 = 6 * 448.
//
// Scale layout (chosen for the GEMM's loads): 256-k panels. Panel p holds, row
// after row, 16 bytes per row: the E4M3 scales of blocks 16p .. 16p+15 in the
// order 0,1,4,5,8,9,12,13, 2,3,6,7,10,11,14,15 (block j at byte
// 8 ((j >> 1) & 1) + 2 (j >> 2) + (j & 1)). A GEMM stage of 256 k then loads a
// tile's scales as one contiguous run, and a matrix-core lane finds the eight
// block scales it needs for the stage in one 8-byte word (see below).
//
// GEMM: the matrix cores of gfx950 scale FP4 operands only by E8M0 powers of
// two per 32 elements, so a 16-element E4M3 scale cannot be applied inside the
// scaled FP4 instruction. Each operand fragment is instead dequantized to fp16
// in registers -- v * s_b is exact in fp16 (2 + 4 significant bits, magnitudes
// 2^-10 .. 2688) -- and multiplied on the fp16 path
// (v_mfma_f32_32x32x16_f16, fp32 accumulation); the product of the two global
// scales multiplies the result once, in the epilogue. A fragment of 8 codes
// costs four v_cvt_scalef32_pk_f16_fp4 (its scale operand contributes only its
// power of two, so it runs with 1.0) and four packed fp16 multiplies by s_b.
// Loads and ring follow the MXFP4 kernel: 256 x 256 workgroup tiles, 256-deep
// K stages in a 2-stage LDS ring filled by direct global->LDS loads, 64-bank
// row swizzle. The eight waves are 2 x 4 of 128 x 64 each (4 x 2 blocks of
// 32 x 32), two per SIMD, so one wave's conversions run under the other's
// MFMAs. In one 64-k step lane l holds
// the 32 codes of k = 32 (l/32) .. +32 of its row (16 bytes); its four
// 16-deep MFMAs take words 0..3 of them, the same words of the A and the W
// lane, so each MFMA sums a consistent set of 16 k and the four together the
// whole step. Words 0, 1 of the lane lie in block 4u + 2 (l/32) of the stage,
// words 2, 3 in the next block: a lane of half h needs blocks 4u + 2h, +1 for
// u = 0..3, bytes 8h .. 8h+7 of its row's panel bytes.
#include <algorithm>

#include "device.h"
#include "launch.h"
#include "quant_common.h"

namespace w4a4 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kQThreads = 256;
constexpr int64_t kMaxGridY = 65535;
constexpr float kE4M3Max = 448.0f;
constexpr float kGlobalDivisor = 2688.0f;   // 6 * 448

// ------------------------------------------------------------- global scale

__global__ void k_zero_word(uint32_t* p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0u;
}

// max |x| as fp16 magnitude bits (an order-preserving integer for finite
// values): each thread one 8-element column chunk over a stride of rows, one
// integer atomic max per workgroup (order-independent result).
__global__ __launch_bounds__(256) void k_absmax_bits(const uint16_t* __restrict__ x, int64_t ldx, int rows,
                                                     int nch, uint32_t* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  uint32_t m = 0;
  if (c < nch) {
    for (int r = blockIdx.y; r < rows; r += gridDim.y) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)r * ldx + 8 * (int64_t)c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(out, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
}

// s_g = fl32(amax / 2688), in place over the magnitude bits.
__global__ void k_global_scale_finish(uint32_t* p) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const float a = __half2float(__ushort_as_half((unsigned short)*p));
  *p = __float_as_uint(a / kGlobalDivisor);
}

// ---------------------------------------------------------------- quantizer

// Lane tile: one 32-element chunk (two blocks) of a row; a wave covers 8 rows x
// the 8 chunks of one 256-k panel, so its 128 scale bytes are one contiguous
// run of the panel; the workgroup's four waves take the next panels of the
// same rows. Row blocks beyond gridDim.y are looped. q16: the code array is
// 16-byte aligned (one store per lane).
__global__ __launch_bounds__(kQThreads) void k_nvfp4_quant(
    const uint16_t* __restrict__ x, int64_t ldx, int rows, int nch, int q16,
    const float* __restrict__ gscale, uint32_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = (blockIdx.x * 4 + wave) * 8 + (lane & 7);     // chunk of the row
  if (c >= nch) return;
  const float sg = *gscale;
  const float d = 6.0f * sg;
  const float nz = opaque_neg_zero();
  const int panel = c >> 3, cp = c & 7;
  // bytes of blocks 2 cp, 2 cp + 1 of the panel row (adjacent in the order above)
  const int spos = 8 * (cp & 1) + 2 * (cp >> 1);
  for (int rb = blockIdx.y; rb * 8 < rows; rb += gridDim.y) {
    const int row = rb * 8 + (lane >> 3);
    if (row >= rows) break;                  // the last row block only
    uint4 raw[4];
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)row * ldx + 32 * (int64_t)c);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = src[i];
    uint32_t w[16];
    words16(raw, w);
    float r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float a = absmax_words<8>(w + 8 * h);
      r[h] = (a == 0.0f) ? 0.0f : fminf(a / d, kE4M3Max);   // d = 0: +inf, saturated
    }
    const uint32_t sb2 = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false) & 0xFFFFu;
    const float S0 = __builtin_amdgcn_cvt_f32_fp8(sb2, 0) * sg;   // fl32(s_b s_g), s_b exact
    const float S1 = __builtin_amdgcn_cvt_f32_fp8(sb2, 1) * sg;
    const float e[2] = {(S0 == 0.0f) ? 0.0f : 1.0f / S0, (S1 == 0.0f) ? 0.0f : 1.0f / S1};
    float t[32];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const h2 v = __builtin_bit_cast(h2, w[k]);
      const float ek = e[k >> 3];
      t[2 * k] = fmaf((float)v.x, ek, nz);        // fl32(x e), sign of x on zero
      t[2 * k + 1] = fmaf((float)v.y, ek, nz);
    }
    const uint4 codes = e2m1_codes32_f32(t);
    const int64_t unit = (int64_t)row * nch + c;   // 16-byte code unit
    if (q16) {
      reinterpret_cast<uint4*>(q)[unit] = codes;
    } else {
      q[4 * unit] = codes.x; q[4 * unit + 1] = codes.y; q[4 * unit + 2] = codes.z; q[4 * unit + 3] = codes.w;
    }
    *reinterpret_cast<uint16_t*>(sc + (int64_t)16 * rows * panel + 16 * (int64_t)row + spos) = (uint16_t)sb2;
  }
}

// --------------------------------------------------------------------- GEMM

struct Params {
  const uint8_t* a;
  const uint8_t* sa;
  const float* ga;
  const uint8_t* w;
  const uint8_t* sw;
  const float* gw;
  int M, N, K;
  void* y;
  int ydtype;
  int64_t ldy;
  int tiles_m, tiles_n;
  int tile_m0, tile_n0;
  int m0, mc, n0, nc;
  int32_t* partials;
};

typedef __attribute__((address_space(3))) void* lds_vptr;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)lds, 16, voff, soff, 0, 0);
}

// 8 codes (one word, element 2i in the low nibble of byte i) times the block
// scale s: the fp16 operand of one 16-deep k-step. Exact.
__device__ __forceinline__ h8 dequant8(uint32_t w, _Float16 s) {
  const h2 ss = {s, s};
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Workgroup tile 256 x 256, waves 2 x 4 (128 x 64 each = 4 x 2 blocks of
// 32 x 32, two waves per SIMD), 256-deep K stages in a 2-stage ring: stage kt + 1 loads while
// stage kt is computed. A stage holds 512 rows of 128 packed bytes (A rows,
// then W rows; each wave-wide 1 KB load covers 8 rows; the 8 16-byte slots of
// a row XOR-swizzled with (row >> 1) & 7 so the 16 lanes reading one slot of
// 16 consecutive rows hit 16 distinct 16-byte bank groups) and the 512 rows'
// 16 panel scale bytes.
template <bool PARTIALS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_nvfp4_gemm(Params p) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4, KB = 256;
  constexpr int NWAVE = WM * WN;
  constexpr int RB = KB / 2;                        // packed bytes per row per stage
  constexpr int SL = RB / 16;                       // 16-byte slots per row
  constexpr int RPK = 1024 / RB;                    // rows per 1 KB load
  constexpr int TI = BM / WM / 32, TJ = BN / WN / 32;
  constexpr int NA = BM / RPK / NWAVE, NW = BN / RPK / NWAVE;
  constexpr int W_OFF = BM * RB;
  constexpr int S_OFF = (BM + BN) * RB;
  constexpr int STAGE = S_OFF + (BM + BN) * 16;
  constexpr int NS = (BM + BN) / 64 / NWAVE;       // 1 KB scale loads per wave per stage
  constexpr int VPM = (TI + TJ) * 8 / (TI * TJ);    // conversion instructions per MFMA
  static_assert(NS * NWAVE * 64 == BM + BN, "scale loads cover the stage's rows");
  __shared__ __align__(16) uint8_t sm0[STAGE];
  __shared__ __align__(16) uint8_t sm1[STAGE];

  const int nblk = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);   // consecutive tiles on one XCD
  constexpr int kGroupRows = 4;
  const int per_group = kGroupRows * p.tiles_n;
  const int grp = bid / per_group;
  const int first_m = grp * kGroupRows;
  const int gsize = min(p.tiles_m - first_m, kGroupRows);
  const int rem = bid - grp * per_group;
  const int tile_m = (p.tile_m0 + first_m + rem % gsize) * BM;
  const int tile_n = (p.tile_n0 + rem / gsize) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int row_bytes = p.K >> 1;
  const int nk = p.K / KB;

  const int a_rows = min(BM, p.M - tile_m), w_rows = min(BN, p.N - tile_n);
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(p.a + (int64_t)tile_m * row_bytes, a_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(p.w + (int64_t)tile_n * row_bytes, w_rows * row_bytes);
  int voffA[NA], voffW[NW];
  const int lrow = lane / SL, lslot = lane % SL;
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = RPK * (wave + NWAVE * i) + lrow;
    voffA[i] = min(row, a_rows - 1) * row_bytes + 16 * (lslot ^ ((row >> 1) & (SL - 1)));
  }
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int row = RPK * (wave + NWAVE * i) + lrow;
    voffW[i] = min(row, w_rows - 1) * row_bytes + 16 * (lslot ^ ((row >> 1) & (SL - 1)));
  }
  // Scales: scale chunk c = NS wave + s holds the 16 panel bytes of 64 rows
  // (A rows 64 c + lane for c < 4, W rows 64 (c - 4) + lane otherwise), stored
  // at LDS scale rows 64 c + lane. A chunk lies wholly in A or in W, so its
  // buffer resource is uniform.
  constexpr int CA = BM / 64;
  int voffS[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = NS * wave + s;
    voffS[s] = 16 * min(64 * (c < CA ? c : c - CA) + lane, (c < CA ? a_rows : w_rows) - 1);
  }

#define ISSUE(KT, SM)                                                                \
  {                                                                                  \
    uint8_t* base_ = (SM);                                                           \
    _Pragma("unroll") for (int i = 0; i < NA; ++i)                                   \
        dma16(rA, voffA[i], (KT) * RB, base_ + (wave + NWAVE * i) * 1024);         \
    _Pragma("unroll") for (int i = 0; i < NW; ++i)                                   \
        dma16(rW, voffW[i], (KT) * RB, base_ + W_OFF + (wave + NWAVE * i) * 1024); \
    _Pragma("unroll") for (int s = 0; s < NS; ++s) {                                 \
      const bool a_ = NS * wave + s < CA;                                            \
      const uint8_t* sb_ = a_ ? p.sa + 16 * ((int64_t)p.M * (KT) + tile_m)           \
                              : p.sw + 16 * ((int64_t)p.N * (KT) + tile_n);          \
      dma16(buffer_rsrc(sb_, 16 * (a_ ? a_rows : w_rows)), voffS[s], 0,              \
            base_ + S_OFF + (NS * wave + s) * 1024);                                 \
    }                                                                                \
  }

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int rowA = wm * (BM / WM) + l32;
  const int rowW = wn * (BN / WN) + l32;
  // The lane's operand slot of step u is 2u + l/32, swizzled; the swizzle only
  // flips address bits 4..6 within the row's 128 bytes, so step u's address is
  // step 0's with bits 5, 6 flipped by u.
  const int offA0 = rowA * RB + 16 * (lhi ^ ((rowA >> 1) & (SL - 1)));
  const int offW0 = rowW * RB + 16 * (lhi ^ ((rowW >> 1) & (SL - 1)));
  uint4 av[1][TI], wv[1][TJ];  // one step's operands: the next step's reads start once these are converted
  uint2 scA[TI], scW[TJ];     // the lane's 8 block-scale bytes of the stage per row block

#define LOAD_OPS(SM, U, B)                                                            \
  {                                                                                  \
    const uint8_t* st_ = (SM);                                                       \
    _Pragma("unroll") for (int i = 0; i < TI; ++i)                                   \
      av[B][i] = *reinterpret_cast<const uint4*>(st_ + (offA0 ^ (32 * (U))) + 32 * RB * i); \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                   \
      wv[B][j] = *reinterpret_cast<const uint4*>(st_ + W_OFF + (offW0 ^ (32 * (U))) + 32 * RB * j); \
  }
#define LOAD_SCALES(SM)                                                              \
  {                                                                                  \
    const uint8_t* ss_ = (SM) + S_OFF + 8 * lhi;                                     \
    _Pragma("unroll") for (int i = 0; i < TI; ++i)                                   \
      scA[i] = *reinterpret_cast<const uint2*>(ss_ + 16 * (rowA + 32 * i));          \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                   \
      scW[j] = *reinterpret_cast<const uint2*>(ss_ + 16 * (BM + rowW + 32 * j));     \
  }
// Matrix work of 64-k step U (a literal) of stage KT: the block scales of the
// step (bytes 2U, 2U + 1 of the lane's 8) as fp16 pairs, then four 16-deep
// MFMAs over words 0..3 of the operands. Once the last words are converted,
// the operand registers are free and step NEXTU's reads from slot SM are
// issued (NEXTU = 4: none), so they overlap the last MFMAs. The partials
// variant runs each 16-element block on its own, with unit scales and only
// the lanes that hold it, so D = sum va vw over that block exactly.
#define MMA_STEP(KT, U, SM, NEXTU)                                                   \
  {                                                                                  \
    constexpr int B = 0;                                                             \
  {                                                                                  \
    if constexpr (PARTIALS) {                                                        \
      for (int hb = 0; hb < 2; ++hb)                                                 \
      for (int bb = 0; bb < 2; ++bb) {                                               \
        const int gblk = 16 * (KT) + 4 * (U) + 2 * hb + bb;                          \
        _Pragma("unroll") for (int i = 0; i < TI; ++i)                               \
        _Pragma("unroll") for (int j = 0; j < TJ; ++j) {                             \
          v16f zacc;                                                                 \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) zacc[r] = 0.0f;             \
          for (int q = 2 * bb; q < 2 * bb + 2; ++q) {                                \
            const _Float16 one_ = (lhi == hb) ? (_Float16)1.0f : (_Float16)0.0f;     \
            zacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(                           \
                dequant8(word_of(av[B][i], q), one_), dequant8(word_of(wv[B][j], q), one_), \
                zacc, 0, 0, 0);                                                      \
          }                                                                          \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) {                           \
            const int m = tile_m + wm * (BM / WM) + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3); \
            const int n = tile_n + wn * (BN / WN) + 32 * j + l32;                     \
            if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)        \
              p.partials[((int64_t)gblk * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] = (int32_t)(zacc[r] * 4.0f); \
          }                                                                          \
        }                                                                            \
      }                                                                              \
      if ((NEXTU) < 4) LOAD_OPS(SM, (NEXTU) & 3, 0);                                 \
    } else {                                                                         \
      h2 fa_[TI], fw_[TJ];                                                           \
      _Pragma("unroll") for (int i = 0; i < TI; ++i)                                 \
        fa_[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((U) < 2 ? scA[i].x : scA[i].y, 1.0f, ((U) & 1) != 0); \
      _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                 \
        fw_[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((U) < 2 ? scW[j].x : scW[j].y, 1.0f, ((U) & 1) != 0); \
      /* two sets of converted fragments: words q + 1 are converted while the */    \
      /* MFMAs of words q run, one MFMA between every four conversions */           \
      h8 a16_[2][TI], w16_[2][TJ];                                                   \
      DEQ(0, 0);                                                                     \
      __builtin_amdgcn_sched_barrier(0);                                             \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                \
        if (q < 3) DEQ((q + 1) & 1, q + 1);                                          \
        if (q == 3 && (NEXTU) < 4) LOAD_OPS(SM, (NEXTU) & 3, 0);                     \
        _Pragma("unroll") for (int i = 0; i < TI; ++i)                               \
        _Pragma("unroll") for (int j = 0; j < TJ; ++j)                               \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a16_[q & 1][i], w16_[q & 1][j], acc[i][j], 0, 0, 0); \
        if (q < 3) {                                                                 \
          _Pragma("unroll") for (int g = 0; g < TI * TJ; ++g) {                      \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   /* one MFMA */     \
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0); /* conversions */  \
          }                                                                          \
        } else if ((NEXTU) < 4) {                                                    \
          _Pragma("unroll") for (int g = 0; g < TI + TJ; ++g) {                      \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   /* one MFMA */     \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   /* one LDS read */ \
          }                                                                          \
        }                                                                            \
        __builtin_amdgcn_sched_barrier(0);                                           \
      }                                                                              \
    }                                                                                \
  }                                                                                  \
  }
// Convert words Q of the step's operands into fragment set SET.
#define DEQ(SET, Q)                                                                  \
  {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < TI; ++i)                                   \
      a16_[SET][i] = dequant8(word_of(av[0][i], (Q)), (Q) < 2 ? fa_[i].x : fa_[i].y); \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                   \
      w16_[SET][j] = dequant8(word_of(wv[0][j], (Q)), (Q) < 2 ? fw_[j].x : fw_[j].y); \
  }
#define PIPE_FENCE() __builtin_amdgcn_sched_barrier(0)
#define STAGE_BARRIER()                                                 \
  {                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                  \
    __builtin_amdgcn_s_barrier();                                       \
    __builtin_amdgcn_sched_barrier(0);                                  \
  }
// Stage KT from slot CUR; stage KT + 1 is issued into NXT (free once every
// wave has passed the barrier) after the first step's operand reads.
#define ITER(KT, CUR, NXT)                                              \
  {                                                                     \
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   /* vmcnt(0) */ \
    STAGE_BARRIER();                                                    \
    LOAD_SCALES(CUR);                                                   \
    LOAD_OPS(CUR, 0, 0);                                                \
    if ((KT) + 1 < nk) ISSUE((KT) + 1, NXT);                            \
    PIPE_FENCE(); MMA_STEP(KT, 0, CUR, 1); PIPE_FENCE();                \
    MMA_STEP(KT, 1, CUR, 2); PIPE_FENCE();                              \
    MMA_STEP(KT, 2, CUR, 3); PIPE_FENCE();                              \
    MMA_STEP(KT, 3, CUR, 4); PIPE_FENCE();                              \
  }

  // Stage pairs with no exit between them (an exit there makes the compiler
  // hold a second copy of the 256 accumulators), then an odd last stage. Each
  // stage names its slot statically, so the compiler tells the loads in flight
  // into one slot from reads of the other and does not wait for them.
  ISSUE(0, sm0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    ITER(kt, sm0, sm1)
    ITER(kt + 1, sm1, sm0)
  }
  if (kt < nk) ITER(kt, sm0, sm1)
#undef ITER
#undef STAGE_BARRIER
#undef PIPE_FENCE
#undef MMA_STEP
#undef DEQ
#undef LOAD_SCALES
#undef LOAD_OPS
#undef ISSUE

  if constexpr (!PARTIALS) {
    const float G = p.ga[0] * p.gw[0];     // fl32(g_a g_w), applied as each value is stored
    // The lane's column and row-half, rebuilt from an operand address that the
    // loop keeps live anyway (offA0 = rowA * 128 + 16 (lhi ^ bit 1 of rowA)),
    // so no lane index has to be held across the loop.
    int oa_ = offA0;
    asm volatile("" : "+v"(oa_));
    const int l32 = (oa_ >> 7) & 31;
    const int lhi = ((oa_ >> 4) ^ (oa_ >> 8)) & 1;
    const int esz = p.ydtype == 0 ? 4 : 2;
    if (a_rows == BM && (int64_t)BM * p.ldy * esz < (int64_t{1} << 31)) {
      // every row valid: buffer stores, row offsets in the scalar offset, lanes
      // with column >= N dropped by the resource's range check
      const int ldb = (int)(p.ldy * esz);
      const __amdgpu_buffer_rsrc_t rY =
          buffer_rsrc(static_cast<uint8_t*>(p.y) + (int64_t)tile_m * ldb, BM * ldb);
      const int row0 = wm * (BM / WM) + 4 * lhi;
      int voffY[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int n = tile_n + wn * (BN / WN) + 32 * j + l32;
        voffY[j] = n < p.N ? row0 * ldb + n * esz : kDroppedOffset;
      }
      if (p.ydtype == 0) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int soff = (32 * i + 8 * (r >> 2) + (r & 3)) * ldb;
#pragma unroll
            for (int j = 0; j < TJ; ++j)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r] * G), rY, voffY[j], soff, kStoreNT);
            __builtin_amdgcn_sched_barrier(0);   // read the accumulators a few at a time
          }
      } else {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int soff = (32 * i + 8 * (r >> 2) + (r & 3)) * ldb;
#pragma unroll
            for (int j = 0; j < TJ; ++j)
              __builtin_amdgcn_raw_buffer_store_b16(__half_as_ushort(__float2half_rn(acc[i][j][r] * G)), rY,
                                                    voffY[j], soff, kStoreNT);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = tile_m + wm * (BM / WM) + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3);
            const int n = tile_n + wn * (BN / WN) + 32 * j + l32;
            if (m < p.M && n < p.N) {
              if (p.ydtype == 0)
                static_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = acc[i][j][r] * G;
              else
                static_cast<__half*>(p.y)[(int64_t)m * p.ldy + n] = __float2half_rn(acc[i][j][r] * G);
            }
          }
    }
  }
}

}  // namespace

void launch_nvfp4_global_scale(const void* x, int64_t rows, int64_t K, int64_t ldx, float* gscale,
                               hipStream_t stream) {
  uint32_t* out = reinterpret_cast<uint32_t*>(gscale);
  hipLaunchKernelGGL(k_zero_word, dim3(1), dim3(64), 0, stream, out);
  if (rows == 0) return;
  const int nch = (int)(K / 8);
  const int gx = (nch + 255) / 256;
  const int gy = (int)std::min<int64_t>(rows, std::max<int64_t>(1, 1024 / gx));
  hipLaunchKernelGGL(k_absmax_bits, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), ldx, (int)rows, nch, out);
  hipLaunchKernelGGL(k_global_scale_finish, dim3(1), dim3(64), 0, stream, out);
}

void launch_nvfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ldx, const float* gscale,
                        uint8_t* q, uint8_t* scales, hipStream_t stream) {
  const int nch = (int)(K / 32);
  const dim3 grid((unsigned)((nch + 31) / 32), (unsigned)std::min<int64_t>((rows + 7) / 8, kMaxGridY));
  const int q16 = (reinterpret_cast<uintptr_t>(q) & 15) == 0;
  hipLaunchKernelGGL(k_nvfp4_quant, grid, dim3(kQThreads), 0, stream, static_cast<const uint16_t*>(x), ldx,
                     (int)rows, nch, q16, gscale, reinterpret_cast<uint32_t*>(q), scales);
}

void launch_nvfp4_gemm(const GemmArgs& g, const float* ga, const float* gw, hipStream_t stream) {
  constexpr int BM = 256, BN = 256;
  Params p;
  p.a = g.a;
  p.sa = static_cast<const uint8_t*>(g.sa);
  p.ga = ga;
  p.w = g.w;
  p.sw = static_cast<const uint8_t*>(g.sw);
  p.gw = gw;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.y = g.y;
  p.ydtype = g.ydtype;
  p.ldy = g.ldy;
  p.m0 = (int)g.m0;
  p.mc = (int)g.mc;
  p.n0 = (int)g.n0;
  p.nc = (int)g.nc;
  p.partials = g.partials;
  p.tile_m0 = (int)(g.m0 / BM);
  p.tile_n0 = (int)(g.n0 / BN);
  p.tiles_m = (int)((g.m0 + g.mc - 1) / BM) - p.tile_m0 + 1;
  p.tiles_n = (int)((g.n0 + g.nc - 1) / BN) - p.tile_n0 + 1;
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  if (g.partials)
    hipLaunchKernelGGL(k_nvfp4_gemm<true>, grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL(k_nvfp4_gemm<false>, grid, dim3(512), 0, stream, p);
}

}  // namespace w4a4
