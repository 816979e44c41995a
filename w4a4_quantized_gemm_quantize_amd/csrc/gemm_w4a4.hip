// W4A4 group-dequantized GEMM for gfx950.
//
// APEX4 ("Efficient Pure W4A4 LLM Inference via Intra-SM Compute
// Rebalancing", abstract): a pure INT4 GEMM on the matrix units, with the
// per-group dequantization done by the vector units -- the cost it identifies
// as the W4A4 bottleneck (its "rho", matrix-unit : vector-unit throughput).
// gfx950 has no INT4 matrix instruction, so packed int4 tiles are staged in LDS
// and widened in registers to int8 for v_mfma_i32_32x32x32_i8:
//   * a packed dword holds 8 codes; (d << 4) & 0xF0F0F0F0 puts the even codes,
//     and d & 0xF0F0F0F0 the odd codes, in the high nibble of each byte, i.e.
//     int8 bytes equal to 16*q (two's complement is preserved). A and W are
//     widened the same way, so every product carries a factor 256 that is
//     folded exactly into the fp32 scale (a power of two) and the k order
//     permutation is the same on both sides.
//   * per block of g = min(group_a, group_w) k values the int32 result is
//     256 * P_b; the epilogue does acc += float(P) * (s_a * s_w / 256) -- one
//     convert, one multiply, one fma per output per group -- then clears P.
//     That is the whole vector-unit cost per output per group; everything
//     else (LDS reads, unpacking) is amortized over a 64 x 64 wave tile.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; tile 128 x 128 outputs,
// K stage 128 (64 packed bytes per row), double-buffered LDS (45 KB), two
// workgroups per CU (2 waves per SIMD) so one wave's epilogue overlaps the
// other's matrix work. Tiles are ordered XCD-contiguous, then in groups of 8
// tile-rows, so workgroups running together on one XCD share A and W slices
// in that XCD's L2.
//
// v_mfma_i32_32x32x32_i8 lane layout: A/B operand lane l holds row (col) l%32
// and 16 consecutive k of chunk l/32; D element r of lane l is
// row 8*(r/4) + 4*(l/32) + r%4, col l%32.
#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int ROW_BYTES = BK / 2;   // packed bytes per row per stage
constexpr int PITCH = 80;           // LDS row pitch: +16 B keeps 16-byte reads conflict-free
constexpr int kThreads = 256;
constexpr int kGroupRows = 8;       // tile-rows per raster group

struct Params {
  const uint8_t* a;
  const float* sa;
  const uint8_t* w;
  const float* sw;
  int ga64, gw64;             // group sizes in units of 64 k
  int gmin;                   // min(ga, gw)
  int M, N, K;
  int ksa, ksw;               // scale columns per row (K / group)
  void* y;
  int ydtype;
  int64_t ldy;
  int tiles_m, tiles_n;       // launch grid in tiles
  int tile_m0, tile_n0;       // first tile of the launch
  int m0, mc, n0, nc;         // partials window
  int32_t* partials;
};

__device__ __forceinline__ v4i widen_x16(uint32_t d0, uint32_t d1) {
  return v4i{(int)((d0 << 4) & 0xF0F0F0F0u), (int)(d0 & 0xF0F0F0F0u),
             (int)((d1 << 4) & 0xF0F0F0F0u), (int)(d1 & 0xF0F0F0F0u)};
}

template <bool PARTIALS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_w4a4_gemm(Params p) {
  __shared__ __align__(16) uint8_t sA[2][BM * PITCH];
  __shared__ __align__(16) uint8_t sW[2][BN * PITCH];
  __shared__ __align__(16) float sSA[2][2][BM];   // [stage][64-k half][row]
  __shared__ __align__(16) float sSW[2][2][BN];

  // ---- tile raster: XCD-contiguous ranges, then groups of kGroupRows tile-rows
  const int nblk = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int per_group = kGroupRows * p.tiles_n;
  const int g = bid / per_group;
  const int first_m = g * kGroupRows;
  const int gsize = min(p.tiles_m - first_m, kGroupRows);
  const int rem = bid - g * per_group;
  const int tm = first_m + rem % gsize;
  const int tn = rem / gsize;
  const int tile_m = (p.tile_m0 + tm) * BM;
  const int tile_n = (p.tile_n0 + tn) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int row_bytes = p.K >> 1;
  const int nk = p.K / BK;

  // ---- global -> LDS staging: 2 x 16 B of A and of W per thread per stage
  const uint8_t* gA[2];
  const uint8_t* gW[2];
  int ldsoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + kThreads * i;
    const int r = idx >> 2, seg = idx & 3;
    gA[i] = p.a + (int64_t)min(tile_m + r, p.M - 1) * row_bytes + seg * 16;
    gW[i] = p.w + (int64_t)min(tile_n + r, p.N - 1) * row_bytes + seg * 16;
    ldsoff[i] = r * PITCH + seg * 16;
  }
  // scales: threads 0..127 stage A-row scales, 128..255 W-row scales
  const bool s_is_a = tid < BM;
  const int srow = s_is_a ? tid : tid - BM;
  const float* gS = s_is_a ? p.sa + (int64_t)min(tile_m + srow, p.M - 1) * p.ksa
                           : p.sw + (int64_t)min(tile_n + srow, p.N - 1) * p.ksw;
  const int s_g64 = s_is_a ? p.ga64 : p.gw64;
  float* sS0 = s_is_a ? &sSA[0][0][srow] : &sSW[0][0][srow];   // [stage][half] stride BM

  uint4 ra0, ra1, rw0, rw1;
  float rs0, rs1;
#define GLOAD(KT)                                                               \
  {                                                                             \
    const int off_ = (KT) * ROW_BYTES;                                          \
    ra0 = *reinterpret_cast<const uint4*>(gA[0] + off_);                        \
    ra1 = *reinterpret_cast<const uint4*>(gA[1] + off_);                        \
    rw0 = *reinterpret_cast<const uint4*>(gW[0] + off_);                        \
    rw1 = *reinterpret_cast<const uint4*>(gW[1] + off_);                        \
    rs0 = gS[(unsigned)(2 * (KT)) / (unsigned)s_g64];                           \
    rs1 = gS[(unsigned)(2 * (KT) + 1) / (unsigned)s_g64];                       \
  }
#define LSTORE(BUF)                                                             \
  {                                                                             \
    *reinterpret_cast<uint4*>(&sA[BUF][ldsoff[0]]) = ra0;                       \
    *reinterpret_cast<uint4*>(&sA[BUF][ldsoff[1]]) = ra1;                       \
    *reinterpret_cast<uint4*>(&sW[BUF][ldsoff[0]]) = rw0;                       \
    *reinterpret_cast<uint4*>(&sW[BUF][ldsoff[1]]) = rw1;                       \
    sS0[(BUF) * 2 * BM] = rs0;                                                  \
    sS0[(BUF) * 2 * BM + BM] = rs1;                                             \
  }

  v16f acc[2][2];
  v16i P[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[i][j][r] = 0.0f;
        P[i][j][r] = 0;
      }
    }

  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  // LDS read offsets (bytes) of this lane's operand rows, without the stage base
  const int offA0 = (wm * 64 + l32) * PITCH + 16 * lhi;
  const int offA1 = offA0 + 32 * PITCH;
  const int offW0 = (wn * 64 + l32) * PITCH + 16 * lhi;
  const int offW1 = offW0 + 32 * PITCH;
  const int k_per_group = p.gmin / BK;    // stages per group when gmin >= 128
  int gcount = 0;                         // stages since the last epilogue
  int gidx = 0;                           // index of the next group to finish

  GLOAD(0);
  LSTORE(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) GLOAD(kt + 1);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(&sA[buf][offA0 + 32 * s2]);
      const uint4 a1 = *reinterpret_cast<const uint4*>(&sA[buf][offA1 + 32 * s2]);
      const uint4 w0 = *reinterpret_cast<const uint4*>(&sW[buf][offW0 + 32 * s2]);
      const uint4 w1 = *reinterpret_cast<const uint4*>(&sW[buf][offW1 + 32 * s2]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v4i av0 = u ? widen_x16(a0.z, a0.w) : widen_x16(a0.x, a0.y);
        const v4i av1 = u ? widen_x16(a1.z, a1.w) : widen_x16(a1.x, a1.y);
        const v4i wv0 = u ? widen_x16(w0.z, w0.w) : widen_x16(w0.x, w0.y);
        const v4i wv1 = u ? widen_x16(w1.z, w1.w) : widen_x16(w1.x, w1.y);
        P[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av0, wv0, P[0][0], 0, 0, 0);
        P[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av0, wv1, P[0][1], 0, 0, 0);
        P[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av1, wv0, P[1][0], 0, 0, 0);
        P[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av1, wv1, P[1][1], 0, 0, 0);
      }
      // A group ends after this 64-k half when gmin == 64, or after the
      // whole stage when the stage completes a group of gmin >= 128.
      bool flush;
      if (p.gmin == 64) {
        flush = true;
      } else {
        flush = (s2 == 1) && (gcount + 1 == k_per_group);
      }
      if (flush) {
        if constexpr (PARTIALS) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int m = tile_m + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
                const int n = tile_n + wn * 64 + j * 32 + l32;
                if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)
                  p.partials[((int64_t)gidx * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] = P[i][j][r] >> 8;
              }
        } else {
          const float* sa_h = &sSA[buf][s2][wm * 64 + 4 * lhi];
          const float* sw_h = &sSW[buf][s2][wn * 64 + l32];
          const float swj0 = sw_h[0] * (1.0f / 256.0f);
          const float swj1 = sw_h[32] * (1.0f / 256.0f);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 sa4 = *reinterpret_cast<const float4*>(sa_h + i * 32 + 8 * q);
              const float sa[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * q + e;
                acc[i][0][r] = fmaf((float)P[i][0][r], sa[e] * swj0, acc[i][0][r]);
                acc[i][1][r] = fmaf((float)P[i][1][r], sa[e] * swj1, acc[i][1][r]);
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) P[i][j][r] = 0;
        ++gidx;
      }
    }
    if (p.gmin != 64) gcount = (gcount + 1 == k_per_group) ? 0 : gcount + 1;
    if (kt + 1 < nk) LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef GLOAD
#undef LSTORE

  if constexpr (!PARTIALS) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = tile_m + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
          const int n = tile_n + wn * 64 + j * 32 + l32;
          if (m < p.M && n < p.N) {
            if (p.ydtype == 0)
              static_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = acc[i][j][r];
            else
              static_cast<__half*>(p.y)[(int64_t)m * p.ldy + n] = __float2half_rn(acc[i][j][r]);
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
  p.ga64 = g.ga / 64;
  p.gw64 = g.gw / 64;
  p.gmin = g.ga < g.gw ? g.ga : g.gw;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.ksa = (int)(g.K / g.ga);
  p.ksw = (int)(g.K / g.gw);
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
    hipLaunchKernelGGL(k_w4a4_gemm<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_w4a4_gemm<false>, grid, dim3(kThreads), 0, stream, p);
}

}  // namespace w4a4
