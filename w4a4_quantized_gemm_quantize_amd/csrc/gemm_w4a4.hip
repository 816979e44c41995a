// W4A4 group-dequantized GEMM for gfx950.
//
// APEX4 ("Efficient Pure W4A4 LLM Inference via Intra-SM Compute
// Rebalancing", abstract): a pure INT4 GEMM on the matrix units, with the
// per-group dequantization done by the vector units -- the cost it identifies
// as the W4A4 bottleneck (its "rho", matrix-unit : vector-unit throughput).
// On gfx950 the vector unit does 64 fp32 lane-ops per clock per CU against
// 4096 int8 MACs on the matrix cores (packed fp32 math is not used), so every
// vector op per output per group matters. Design:
//
//   * gfx950 has no INT4 matrix instruction. Packed int4 tiles are fetched
//     from HBM/L2 and widened ONCE per workgroup, by the threads that stage
//     them, into int8 operands in LDS: for a packed dword d (8 codes),
//     (d << 4) & 0xF0F0F0F0 puts the even codes and d & 0xF0F0F0F0 the odd
//     codes in the high nibble of each byte, i.e. int8 bytes equal to 16*q
//     (two's complement preserved). A and W are widened the same way, so each
//     product carries a factor 256, folded exactly into the fp32 scale (a power
//     of two), and the k permutation is the same on both sides.
//   * The waves read MFMA-ready 16-byte operands from LDS and run
//     v_mfma_i32_32x32x32_i8. A group's partial P_b (times 256) starts from an
//     inline zero accumulator, so clearing it costs nothing.
//   * Epilogue per output per group: acc += float(P) * (s_a * s_w / 256) --
//     one convert, one multiply, one fma, the minimum for an int32 partial
//     and two fp32 scales.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; tile 128 x 128 outputs,
// K stage 128, double-buffered LDS (76 KB), two workgroups per CU (2 waves per
// SIMD) so one wave's epilogue overlaps the other's matrix work. Tiles are
// ordered XCD-contiguous, then in groups of 8 tile-rows, so workgroups running
// together on one XCD share A and W slices in that XCD's L2.
//
// v_mfma_i32_32x32x32_i8 lane layout: A/B operand lane l holds row (col) l%32
// and 16 k of chunk l/32; D element r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
// col l%32.
#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int ROW_BYTES = BK / 2;   // packed bytes per row per stage
constexpr int PITCH = 144;          // LDS bytes per row: 128 int8 + 16 pad (conflict-free 16 B reads)
constexpr int kThreads = 256;
constexpr int kGroupRows = 8;       // tile-rows per raster group

// Group modes: epilogue after every 64-k half (g = 64), after every stage
// (g = 128), or after several stages (g > 128).
enum { G64 = 0, G128 = 1, GBIG = 2 };

struct Params {
  const uint8_t* a;
  const float* sa;
  const uint8_t* w;
  const float* sw;
  int sha, shw;               // scale column of 64-k half h = h >> sh (31: one column)
  int stages_per_group;       // GBIG only
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

__device__ __forceinline__ uint32_t even16(uint32_t d) { return (d << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t odd16(uint32_t d) { return d & 0xF0F0F0F0u; }

// 32 packed codes (16 B) -> two 16-byte int8 operand pieces in LDS.
__device__ __forceinline__ void widen_store(uint8_t* dst, uint4 v) {
  *reinterpret_cast<uint4*>(dst) = uint4{even16(v.x), odd16(v.x), even16(v.y), odd16(v.y)};
  *reinterpret_cast<uint4*>(dst + 16) = uint4{even16(v.z), odd16(v.z), even16(v.w), odd16(v.w)};
}

__device__ __forceinline__ v4i as_v4i(uint4 v) { return v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}; }

template <bool PARTIALS, int MODE>
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
  const int grp = bid / per_group;
  const int first_m = grp * kGroupRows;
  const int gsize = min(p.tiles_m - first_m, kGroupRows);
  const int rem = bid - grp * per_group;
  const int tile_m = (p.tile_m0 + first_m + rem % gsize) * BM;
  const int tile_n = (p.tile_n0 + rem / gsize) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int row_bytes = p.K >> 1;
  const int nk = p.K / BK;

  // ---- staging: each thread fetches 2 x 16 B of A and of W per stage
  const uint8_t* gA0 = p.a + (int64_t)min(tile_m + (tid >> 2), p.M - 1) * row_bytes + (tid & 3) * 16;
  const uint8_t* gA1 = p.a + (int64_t)min(tile_m + 64 + (tid >> 2), p.M - 1) * row_bytes + (tid & 3) * 16;
  const uint8_t* gW0 = p.w + (int64_t)min(tile_n + (tid >> 2), p.N - 1) * row_bytes + (tid & 3) * 16;
  const uint8_t* gW1 = p.w + (int64_t)min(tile_n + 64 + (tid >> 2), p.N - 1) * row_bytes + (tid & 3) * 16;
  const int st0 = (tid >> 2) * PITCH + (tid & 3) * 32;
  const int st1 = st0 + 64 * PITCH;
  // scales: threads 0..127 stage A-row scales, 128..255 W-row scales
  const bool s_is_a = tid < BM;
  const int srow = s_is_a ? tid : tid - BM;
  const float* gS = s_is_a ? p.sa + (int64_t)min(tile_m + srow, p.M - 1) * p.ksa
                           : p.sw + (int64_t)min(tile_n + srow, p.N - 1) * p.ksw;
  const int ssh = s_is_a ? p.sha : p.shw;
  float* sS = s_is_a ? &sSA[0][0][srow] : &sSW[0][0][srow];

  uint4 ra0, ra1, rw0, rw1;
  float rs0, rs1;
#define GLOAD(KT)                                                     \
  {                                                                   \
    const int off_ = (KT) * ROW_BYTES;                                \
    ra0 = *reinterpret_cast<const uint4*>(gA0 + off_);                \
    ra1 = *reinterpret_cast<const uint4*>(gA1 + off_);                \
    rw0 = *reinterpret_cast<const uint4*>(gW0 + off_);                \
    rw1 = *reinterpret_cast<const uint4*>(gW1 + off_);                \
    rs0 = gS[(2 * (KT)) >> ssh];                                      \
    rs1 = gS[(2 * (KT) + 1) >> ssh];                                  \
  }
#define LSTORE(BUF)                                                   \
  {                                                                   \
    widen_store(&sA[BUF][st0], ra0);                                  \
    widen_store(&sA[BUF][st1], ra1);                                  \
    widen_store(&sW[BUF][st0], rw0);                                  \
    widen_store(&sW[BUF][st1], rw1);                                  \
    sS[(BUF) * 2 * BM] = rs0;                                         \
    sS[(BUF) * 2 * BM + BM] = rs1;                                    \
  }

  v16f acc[2][2];
  v16i P[2][2];
  const v16i zero16 = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  const v32f zero32 = {};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      P[i][j] = zero16;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }

  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int rdA = (wm * 64 + l32) * PITCH + 16 * lhi;   // + i*32*PITCH + 32*s
  const int rdW = (wn * 64 + l32) * PITCH + 16 * lhi;
  int gcount = 0;     // GBIG: stages accumulated into P since the last epilogue
  int gidx = 0;       // index of the next group to finish (partials export)

  GLOAD(0);
  LSTORE(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) GLOAD(kt + 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4i a0 = as_v4i(*reinterpret_cast<const uint4*>(&sA[buf][rdA + 32 * s]));
      const v4i a1 = as_v4i(*reinterpret_cast<const uint4*>(&sA[buf][rdA + 32 * PITCH + 32 * s]));
      const v4i w0 = as_v4i(*reinterpret_cast<const uint4*>(&sW[buf][rdW + 32 * s]));
      const v4i w1 = as_v4i(*reinterpret_cast<const uint4*>(&sW[buf][rdW + 32 * PITCH + 32 * s]));
      // first k-step of a group starts from an inline zero accumulator
      const bool fresh = (MODE == G64) ? (s == 0 || s == 2) : (MODE == G128) ? (s == 0) : false;
      if (fresh) {
        P[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, w0, zero16, 0, 0, 0);
        P[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, w1, zero16, 0, 0, 0);
        P[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, w0, zero16, 0, 0, 0);
        P[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, w1, zero16, 0, 0, 0);
      } else {
        P[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, w0, P[0][0], 0, 0, 0);
        P[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, w1, P[0][1], 0, 0, 0);
        P[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, w0, P[1][0], 0, 0, 0);
        P[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, w1, P[1][1], 0, 0, 0);
      }
      bool flush;
      if (MODE == G64) flush = (s == 1 || s == 3);
      else if (MODE == G128) flush = (s == 3);
      else flush = (s == 3) && (gcount + 1 == p.stages_per_group);
      if (flush) {
        const int h = s >> 1;   // 64-k half whose scales apply
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
          // Scale products t[m][n] = s_a[m] * s_w[n] / 256 as a rank-1 matrix
          // product on the matrix cores: one two-block 32x32x1 fp32 MFMA gives
          // the 32x32 tiles (i = 0, j) and (i = 1, j), in the same lane/register
          // layout as the int32 partials. Lane l supplies row l of the wave's 64
          // A rows (block l / 32) and column 32 j + l % 32 of its W columns.
          const float av = sSA[buf][h][wm * 64 + lane];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float bv = sSW[buf][h][wn * 64 + 32 * j + l32] * (1.0f / 256.0f);
            const v32f T = __builtin_amdgcn_mfma_f32_32x32x1f32(av, bv, zero32, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc[0][j][r] = fmaf((float)P[0][j][r], T[r], acc[0][j][r]);
              acc[1][j][r] = fmaf((float)P[1][j][r], T[16 + r], acc[1][j][r]);
            }
          }
        }
        if (MODE == GBIG) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) P[i][j] = zero16;
        }
        ++gidx;
      }
    }
    if (MODE == GBIG) gcount = (gcount + 1 == p.stages_per_group) ? 0 : gcount + 1;
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

// log2(group / 64) for a power-of-two group, 31 (a single column) for group == K.
int scale_shift(int64_t group, int64_t K) {
  if (group == K && (group & (group - 1))) return 31;
  int s = 0;
  while ((64LL << s) < group) ++s;
  return s;
}

template <bool PARTIALS>
void launch_mode(int mode, const Params& p, dim3 grid, hipStream_t stream) {
  switch (mode) {
    case G64: hipLaunchKernelGGL((k_w4a4_gemm<PARTIALS, G64>), grid, dim3(kThreads), 0, stream, p); return;
    case G128: hipLaunchKernelGGL((k_w4a4_gemm<PARTIALS, G128>), grid, dim3(kThreads), 0, stream, p); return;
    default: hipLaunchKernelGGL((k_w4a4_gemm<PARTIALS, GBIG>), grid, dim3(kThreads), 0, stream, p); return;
  }
}

}  // namespace

void launch_w4a4_gemm(const GemmArgs& g, hipStream_t stream) {
  Params p;
  p.a = g.a;
  p.sa = static_cast<const float*>(g.sa);
  p.w = g.w;
  p.sw = static_cast<const float*>(g.sw);
  p.sha = scale_shift(g.ga, g.K);
  p.shw = scale_shift(g.gw, g.K);
  const int64_t gmin = g.ga < g.gw ? g.ga : g.gw;
  const int mode = gmin == 64 ? G64 : gmin == 128 ? G128 : GBIG;
  p.stages_per_group = (int)(gmin / BK);
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
    launch_mode<true>(mode, p, grid, stream);
  else
    launch_mode<false>(mode, p, grid, stream);
}

}  // namespace w4a4
