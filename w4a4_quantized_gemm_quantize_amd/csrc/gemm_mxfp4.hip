// MXFP4 GEMM for gfx950 on the block-scaled FP4 matrix-core path.
//
// MXFP4 = FP4 E2M1 elements with one E8M0 scale per 32 along K (the
// "open-standard MXFP4" of the FP4 RL abstract; block rule of OCP MX v1.0).
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operand formats set to FP4
// multiplies a 16 x 128 A tile by a 128 x 16 B tile; each lane supplies 32
// consecutive K codes of one row (16 bytes) and the E8M0 byte of exactly that
// 32-block, so the block scales are applied inside the instruction and the
// accumulation is fp32 with no vector-unit epilogue.
//
// Tile: 128 x 128 per 256-thread workgroup (2 x 2 waves of 64 x 64), K step
// 128 (one MFMA per 16 x 16 block per step), double-buffered LDS.
#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int ROW_BYTES = BK / 2;
constexpr int LDS_STRIDE = ROW_BYTES + 16;
constexpr int kThreads = 256;
constexpr int kFmtFp4 = 4;       // cbsz / blgp operand format code for FP4 E2M1
constexpr int kUnitScale = 127;  // E8M0 byte of 2^0

struct Params {
  const uint8_t* a;
  const uint8_t* ea;
  const uint8_t* w;
  const uint8_t* ew;
  int64_t M, N, K;
  void* y;
  int ydtype;
  int64_t ldy;
  int64_t tile_m0, tile_n0;
  int64_t m0, mc, n0, nc;
  int32_t* partials;
};

__device__ __forceinline__ v8i as_operand(uint4 v) {
  return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

template <bool PARTIALS>
__global__ __launch_bounds__(kThreads) void k_mxfp4_gemm(Params p) {
  __shared__ __align__(16) uint8_t sA[2][BM * LDS_STRIDE];
  __shared__ __align__(16) uint8_t sW[2][BN * LDS_STRIDE];
  __shared__ uint32_t sEA[2][BM];   // 4 scale bytes (the 4 blocks of a K step)
  __shared__ uint32_t sEW[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tile_m = (p.tile_m0 + blockIdx.y) * BM;
  const int64_t tile_n = (p.tile_n0 + blockIdx.x) * BN;
  const int64_t row_bytes = p.K / 2;
  const int64_t row_scales = p.K / 32;
  const int nk = (int)(p.K / BK);

  const uint8_t* ga_ptr[2];
  const uint8_t* gw_ptr[2];
  int lds_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + kThreads * i;
    const int r = idx >> 2, seg = idx & 3;
    ga_ptr[i] = p.a + min(tile_m + r, p.M - 1) * row_bytes + seg * 16;
    gw_ptr[i] = p.w + min(tile_n + r, p.N - 1) * row_bytes + seg * 16;
    lds_off[i] = r * LDS_STRIDE + seg * 16;
  }
  const bool scale_is_a = tid < BM;
  const int srow = scale_is_a ? tid : tid - BM;
  const uint8_t* sptr = scale_is_a ? p.ea + min(tile_m + srow, p.M - 1) * row_scales
                                   : p.ew + min(tile_n + srow, p.N - 1) * row_scales;

  uint4 ra[2], rw[2];
  uint32_t rs;
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = *reinterpret_cast<const uint4*>(ga_ptr[i] + (int64_t)kt * ROW_BYTES);
      rw[i] = *reinterpret_cast<const uint4*>(gw_ptr[i] + (int64_t)kt * ROW_BYTES);
    }
    rs = *reinterpret_cast<const uint32_t*>(sptr + (int64_t)kt * 4);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4*>(&sA[buf][lds_off[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&sW[buf][lds_off[i]]) = rw[i];
    }
    if (scale_is_a) sEA[buf][srow] = rs;
    else sEW[buf][srow] = rs;
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15;
  const int lblk = lane >> 4;     // which 32-block of the K step this lane holds
  const int orow = (lane >> 4) * 4;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    v8i a[4], b[4];
    int ea[4], eb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + lrow;
      a[i] = as_operand(*reinterpret_cast<const uint4*>(&sA[buf][r * LDS_STRIDE + lblk * 16]));
      ea[i] = (int)((sEA[buf][r] >> (8 * lblk)) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + j * 16 + lrow;
      b[j] = as_operand(*reinterpret_cast<const uint4*>(&sW[buf][r * LDS_STRIDE + lblk * 16]));
      eb[j] = (int)((sEW[buf][r] >> (8 * lblk)) & 0xFFu);
    }
    if constexpr (PARTIALS) {
      // One 32-block at a time: only the lanes holding block q keep their
      // codes, scales are 2^0, and D = sum va*vw over that block exactly.
      const v8i zero = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t blk = (int64_t)kt * 4 + q;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                lblk == q ? a[i] : zero, lblk == q ? b[j] : zero, v4f{0.f, 0.f, 0.f, 0.f},
                kFmtFp4, kFmtFp4, 0, kUnitScale, 0, kUnitScale);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int64_t m = tile_m + wm * 64 + i * 16 + orow + r;
              const int64_t n = tile_n + wn * 64 + j * 16 + lrow;
              if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)
                p.partials[(blk * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] = (int32_t)(d[r] * 4.0f);
            }
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a[i], b[j], acc[i][j], kFmtFp4, kFmtFp4, 0, ea[i], 0, eb[j]);
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

void launch_mxfp4_gemm(const GemmArgs& g, hipStream_t stream) {
  Params p;
  p.a = g.a;
  p.ea = static_cast<const uint8_t*>(g.sa);
  p.w = g.w;
  p.ew = static_cast<const uint8_t*>(g.sw);
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
    hipLaunchKernelGGL(k_mxfp4_gemm<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_mxfp4_gemm<false>, grid, dim3(kThreads), 0, stream, p);
}

}  // namespace w4a4
