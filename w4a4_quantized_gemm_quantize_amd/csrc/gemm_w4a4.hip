// W4A4 group-dequantized GEMM for gfx950.
//
// APEX4 ("Efficient Pure W4A4 LLM Inference via Intra-SM Compute
// Rebalancing", abstract): a pure INT4 GEMM on the matrix units, with the
// per-group dequantization done by the vector units -- the cost it identifies
// as the W4A4 bottleneck. gfx950 has no INT4 matrix instruction, so packed
// int4 tiles are staged in LDS and widened in registers to int8 for
// v_mfma_i32_16x16x64_i8:
//   * a packed dword holds 8 codes; (d << 4) & 0xF0F0F0F0 puts the even codes,
//     and d & 0xF0F0F0F0 the odd codes, in the high nibble of each byte, i.e.
//     int8 bytes equal to 16*q (two's complement is preserved). A and W are
//     widened the same way, so every product carries a factor 256 that is
//     folded exactly into the fp32 scale (a power of two) and the k order
//     permutation is the same on both sides.
//   * per block of g = min(group_a, group_w) k values the int32 result is
//     P_b * 256; the epilogue does acc += (s_a * s_w / 256) * float(P),
//     all in fp32 registers, then clears P.
//
// Tile: 128 x 128 outputs per 256-thread workgroup (2 x 2 waves of 64 x 64,
// each a 4 x 4 grid of 16 x 16 MFMA blocks), K step 128, double-buffered LDS.
// MFMA 16x16 output layout: lane l, element r -> row 4*(l/16) + r, col l%16.
#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int ROW_BYTES = BK / 2;            // packed bytes per row per K step
constexpr int LDS_STRIDE = ROW_BYTES + 16;   // padded row pitch in LDS
constexpr int kThreads = 256;

struct Params {
  const uint8_t* a;
  const float* sa;
  const uint8_t* w;
  const float* sw;
  int ga, gw, gmin;
  int64_t M, N, K;
  void* y;
  int ydtype;
  int64_t ldy;
  int64_t tile_m0, tile_n0;   // first tile (in tiles) of the launch
  int64_t m0, mc, n0, nc;     // partials window
  int32_t* partials;
};

__device__ __forceinline__ v4i widen_x16(uint2 p) {
  v4i r;
  r[0] = (int)((p.x << 4) & 0xF0F0F0F0u);
  r[1] = (int)(p.x & 0xF0F0F0F0u);
  r[2] = (int)((p.y << 4) & 0xF0F0F0F0u);
  r[3] = (int)(p.y & 0xF0F0F0F0u);
  return r;
}

template <bool PARTIALS>
__global__ __launch_bounds__(kThreads) void k_w4a4_gemm(Params p) {
  __shared__ __align__(16) uint8_t sA[2][BM * LDS_STRIDE];
  __shared__ __align__(16) uint8_t sW[2][BN * LDS_STRIDE];
  __shared__ __align__(16) float sSA[2][2][BM];
  __shared__ __align__(16) float sSW[2][2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tile_m = (p.tile_m0 + blockIdx.y) * BM;
  const int64_t tile_n = (p.tile_n0 + blockIdx.x) * BN;
  const int64_t row_bytes = p.K / 2;
  const int nk = (int)(p.K / BK);

  // Global -> register staging: 2 x 16 B of A and of W per thread.
  const uint8_t* ga_ptr[2];
  const uint8_t* gw_ptr[2];
  int lds_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + kThreads * i;
    const int r = idx >> 2, seg = idx & 3;
    const int64_t am = min(tile_m + r, p.M - 1);
    const int64_t wn_ = min(tile_n + r, p.N - 1);
    ga_ptr[i] = p.a + am * row_bytes + seg * 16;
    gw_ptr[i] = p.w + wn_ * row_bytes + seg * 16;
    lds_off[i] = r * LDS_STRIDE + seg * 16;
  }
  // Scale staging: threads 0..127 fetch A-row scales, 128..255 W-row scales.
  const bool scale_is_a = tid < BM;
  const int srow = scale_is_a ? tid : tid - BM;
  const float* sptr = scale_is_a ? p.sa + min(tile_m + srow, p.M - 1) * (p.K / p.ga)
                                 : p.sw + min(tile_n + srow, p.N - 1) * (p.K / p.gw);
  const int sgroup = scale_is_a ? p.ga : p.gw;

  uint4 ra[2], rw[2];
  float rs[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = *reinterpret_cast<const uint4*>(ga_ptr[i] + (int64_t)kt * ROW_BYTES);
      rw[i] = *reinterpret_cast<const uint4*>(gw_ptr[i] + (int64_t)kt * ROW_BYTES);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) rs[h] = sptr[((int64_t)kt * BK + 64 * h) / sgroup];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4*>(&sA[buf][lds_off[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&sW[buf][lds_off[i]]) = rw[i];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (scale_is_a) sSA[buf][h][srow] = rs[h];
      else sSW[buf][h][srow] = rs[h];
    }
  };

  v4f acc[4][4];
  v4i P[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      P[i][j] = v4i{0, 0, 0, 0};
    }

  const int lrow = lane & 15;          // row (A) / col (W) inside a 16-block
  const int lchunk = lane >> 4;        // which 8-byte chunk of a 32-byte half
  const int orow = (lane >> 4) * 4;    // first output row of this lane in a block

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i a8[4], b8[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = (wm * 64 + i * 16 + lrow) * LDS_STRIDE + h * 32 + lchunk * 8;
        a8[i] = widen_x16(*reinterpret_cast<const uint2*>(&sA[buf][off]));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = (wn * 64 + j * 16 + lrow) * LDS_STRIDE + h * 32 + lchunk * 8;
        b8[j] = widen_x16(*reinterpret_cast<const uint2*>(&sW[buf][off]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          P[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a8[i], b8[j], P[i][j], 0, 0, 0);

      const int64_t kend = (int64_t)kt * BK + 64 * (h + 1);
      if (kend % p.gmin == 0) {
        if constexpr (PARTIALS) {
          const int64_t b = kend / p.gmin - 1;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int64_t m = tile_m + wm * 64 + i * 16 + orow + r;
                const int64_t n = tile_n + wn * 64 + j * 16 + lrow;
                if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)
                  p.partials[(b * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] = P[i][j][r] >> 8;
              }
        } else {
          float sw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) sw[j] = sSW[buf][h][wn * 64 + j * 16 + lrow] * (1.0f / 256.0f);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 sa4 = *reinterpret_cast<const float4*>(&sSA[buf][h][wm * 64 + i * 16 + orow]);
            const float sa[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[i][j][r] = fmaf((float)P[i][j][r], sa[r] * sw[j], acc[i][j][r]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) P[i][j] = v4i{0, 0, 0, 0};
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  if constexpr (!PARTIALS) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = tile_m + wm * 64 + i * 16 + orow + r;
          const int64_t n = tile_n + wn * 64 + j * 16 + lrow;
          if (m < p.M && n < p.N) {
            if (p.ydtype == 0)
              static_cast<float*>(p.y)[m * p.ldy + n] = acc[i][j][r];
            else
              static_cast<__half*>(p.y)[m * p.ldy + n] = __float2half_rn(acc[i][j][r]);
          }
        }
  }
}

}  // namespace

void launch_w4a4_gemm(const GemmArgs& g, hipStream_t stream) {
  Params p;
  p.a = g.a;
  p.sa = static_cast<const float*>(g.sa);
  p.w = g.w;
  p.sw = static_cast<const float*>(g.sw);
  p.ga = g.ga;
  p.gw = g.gw;
  p.gmin = g.ga < g.gw ? g.ga : g.gw;
  p.M = g.M;
  p.N = g.N;
  p.K = g.K;
  p.y = g.y;
  p.ydtype = g.ydtype;
  p.ldy = g.ldy;
  p.m0 = g.m0;
  p.mc = g.mc;
  p.n0 = g.n0;
  p.nc = g.nc;
  p.partials = g.partials;
  p.tile_m0 = g.m0 / BM;
  p.tile_n0 = g.n0 / BN;
  const int64_t tiles_m = (g.m0 + g.mc - 1) / BM - p.tile_m0 + 1;
  const int64_t tiles_n = (g.n0 + g.nc - 1) / BN - p.tile_n0 + 1;
  const dim3 grid((unsigned)tiles_n, (unsigned)tiles_m);
  if (g.partials)
    hipLaunchKernelGGL(k_w4a4_gemm<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_w4a4_gemm<false>, grid, dim3(kThreads), 0, stream, p);
}

}  // namespace w4a4
