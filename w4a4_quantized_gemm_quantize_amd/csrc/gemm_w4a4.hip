// W4A4 group-dequantized GEMM for gfx950.
//
// APEX4 ("Efficient Pure W4A4 LLM Inference via Intra-SM Compute
// Rebalancing", abstract): a pure INT4 GEMM on the matrix units, with the
// per-group dequantization done by the vector units -- the cost it identifies
// as the W4A4 bottleneck (its "rho", matrix-unit : vector-unit throughput).
// On gfx950 the vector unit does 64 fp32 lane-ops per clock per CU against
// 8192 6-bit MACs on the matrix cores (packed fp32 math is not used), so the
// design moves every piece of the dequantization it can onto the matrix cores
// and keeps the vector work per output per group at ONE fma:
//
//   * gfx950 has no INT4 matrix instruction, but FP6 E2M3 holds every INT4
//     code exactly: the field [sign 00 m] is the subnormal +-m/8, and the FP6
//     path of the matrix cores runs at the FP4 rate, twice the FP8/INT8 rate.
//     The codes are stored 4 bits each in a layout folded from that 6-bit
//     stream (see the C header), so the threads that stage a tile rebuild the
//     operand stream with two ANDs and one AND-OR per 16 codes, ONCE per
//     workgroup, into LDS.
//   * v_mfma_scale_f32_32x32x64_f8f6f4 multiplies them with an E8M0 scale of
//     2^3 per operand, so each partial P_b = sum qa*qw comes out as an exact
//     integer in fp32 (|P_b| <= 49 g < 2^24) -- no int->float convert.
//   * The scale product t[m][n] = s_a[m] * s_w[n] is a rank-1 matrix: one
//     two-block 32x32x1 fp32 MFMA gives it for two 32x32 tiles, in the lane
//     layout of the partials.
//   * Epilogue per output per group: acc = fma(P, t, acc).
//
// Workgroup: TM x 128 output tile, 2 TM threads = TM / 32 waves in a
// (TM / 64) x 2 grid of 64 x 64, K stage 128 (two MFMA k-steps),
// double-buffered LDS. TM = 256 (82 KB, one workgroup per CU) stages a
// quarter fewer rows per MAC than TM = 128 (50 KB, two per CU), which serves
// M <= 128, where a 256-row tile would be half empty. Either way two waves per
// SIMD. The staging threads fetch stage kt+2 while
// stage kt is computed and stage kt+1 is unpacked (two register sets), and the
// stage barrier orders LDS only, so no wait drains those loads.
// With g = 128 a stage is one group and runs as a software pipeline of ten
// chunks, each one MFMA issued first and then the vector work that runs under
// it: the epilogue of a tile whose partials finished two or more MFMAs
// earlier (so it never waits on the matrix core), one of the staging stores
// of the next stage, or operand reads for the next chunks -- spread so that
// the LDS queue never takes a burst. The last two tiles' epilogues run under
// the next stage's first four MFMAs (their partials and scale product carried
// over); empty asm statements pin each MFMA, and scheduling barriers keep
// each chunk's work in the chunk. Other group sizes run each stage's MFMAs,
// then its epilogues. Tiles are ordered XCD-contiguous, then in
// groups of 8 tile-rows, so workgroups running together on one XCD share A and
// W slices in that XCD's L2.
//
// 32x32 MFMA lane layout: operand lane l holds row (col) l%32 and the k-chunk
// l/32 (32 consecutive k: 24 bytes of FP6 fields, field i at bits 6i);
// result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, col l%32
// (block b of the two-block fp32 MFMA in registers 16b .. 16b+15, with operand
// lanes 32b .. 32b+31).
#include <algorithm>

#include "device.h"
#include "launch.h"
#include "quant_common.h"

namespace w4a4 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int BN = 128, BK = 128;
constexpr int ROW_BYTES = BK / 2;   // packed bytes per row per stage
// LDS row of one 128-k stage: four 32-code FP6 operand chunks of 24 bytes,
// each split into a 16-byte main part and an 8-byte tail, kept in two arrays
// so every read is naturally aligned. The LDS serves 16 lanes of 16-byte (32
// lanes of 8-byte) accesses per clock over 64 banks: readers take one chunk
// of 16 (32) consecutive rows, writers 4 chunks of 4 (8) rows. Unpadded rows
// with the chunk index XOR-swizzled by (row >> 2) & 3 (main) and (row >> 3) & 3
// (tail) put both patterns in distinct banks.
constexpr int PM = 64;              // main part: 4 x 16 B
constexpr int PT = 32;              // tail part: 4 x 8 B
__device__ __forceinline__ int main_off(int row, int chunk) { return row * PM + 16 * (chunk ^ ((row >> 2) & 3)); }
__device__ __forceinline__ int tail_off(int row, int chunk) { return row * PT + 8 * (chunk ^ ((row >> 3) & 3)); }
constexpr int kGroupRows = 8;       // tile-rows per raster group
constexpr int kUnitScale = 127 + 3; // E8M0 2^3: FP6 E2M3 [s 00 m] = +-m/8, times 2^3 = +-m
constexpr int kFmtFp6 = 2;          // cbsz / blgp operand format code for FP6 E2M3

// Group modes: epilogue after every 64-k step (g = 64), after every stage
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
  int ksa, ksw;               // scale groups per row (K / group); scales are group-major [K/group][rows]
  void* y;
  int ydtype;
  int64_t ldy;
  int tiles_m, tiles_n;       // launch grid in tiles
  int tile_m0, tile_n0;       // first tile of the launch
  int m0, mc, n0, nc;         // partials window
  int32_t* partials;
  int stages_per_split;       // K split: workgroup b takes stages [s S, (s+1) S), s = b / tiles
  int64_t split_stride;       // elements between the splits' outputs (0: no split)
};

// Folding masks of the packed INT4 unit (see the C header): X carries the
// stream's first word S0 and, at positions 3, 4 mod 6 (kFoldX), bits of S1; Y
// carries S2 and, at positions 0, 5 mod 6 (kFoldY), the rest of S1.
constexpr uint32_t kFoldX = 0x18618618u;
constexpr uint32_t kFoldY = 0x61861861u;

// 32 packed codes (16 B = two units X0 Y0 X1 Y1) -> their 192-bit FP6 E2M3
// operand stream S0..S5 in LDS: S0..S3 to the main part, S4, S5 to the tail.
__device__ __forceinline__ void unpack_store(uint8_t* dm, uint8_t* dt, uint4 v) {
  const uint32_t s1 = (v.x & kFoldX) | (v.y & kFoldY);
  const uint32_t s4 = (v.z & kFoldX) | (v.w & kFoldY);
  *reinterpret_cast<uint4*>(dm) = uint4{v.x & ~kFoldX, s1, v.y & ~kFoldY, v.z & ~kFoldX};
  *reinterpret_cast<uint2*>(dt) = uint2{s4, v.w & ~kFoldY};
}

// The 6 FP6 words of one lane's operand (row l%32, k-chunk l/32) from LDS. In
// FP6 mode the instruction reads registers 0..5 of the operand, so 6 and 7 are
// left undefined (no register moves to clear them).
__device__ __forceinline__ v8i load_op(const uint8_t* pm, const uint8_t* pt) {
  const v4i x = *reinterpret_cast<const v4i*>(pm);
  const v2i y = *reinterpret_cast<const v2i*>(pt);
  const v4i y4 = __builtin_shufflevector(y, y, 0, 1, -1, -1);
  return __builtin_shufflevector(x, y4, 0, 1, 2, 3, 4, 5, -1, -1);
}

// Workgroup barrier that orders LDS only: __syncthreads() would also wait for
// every global load in flight, i.e. for the prefetch of later stages.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct GroupScales {
  v32f t;          // s_a x s_w for two 32x32 tiles (unused with per-row A scales)
  float sw0, sw1;  // the lane's W scales of column blocks 0 and 1 (per-row A scales)
};

__device__ __forceinline__ uint4 as_uint4(v4u v) { return uint4{v.x, v.y, v.z, v.w}; }

__device__ __forceinline__ v16f mma(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kFmtFp6, kFmtFp6, 0, kUnitScale, 0, kUnitScale);
}

// ROWA: one activation scale per row (group_a == K, the per-token end of the
// mixed-granularity mode). Then s_a[m] is common to every group and factors
// out of the sum: the epilogue is acc = fma(P, s_w[n], acc) with s_w[n] a
// per-lane constant (no scale-product MFMA) and the store multiplies by s_a[m].
template <bool PARTIALS, int MODE, bool ROWA, int TM>
__global__ __launch_bounds__(2 * TM) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_w4a4_gemm(Params p) {
  static_assert(TM == 128 || TM == 256, "tile heights");
  constexpr int BM = TM, kThreads = 2 * TM;
  constexpr int HALF = TM / 2;          // A rows staged per thread: r, r + HALF
  constexpr bool W2 = TM == 128;        // W rows staged per thread: r (and r + 64)
  __shared__ __align__(16) uint8_t sA[2][BM * PM];   // FP6 operand main parts
  __shared__ __align__(16) uint8_t sW[2][BN * PM];
  __shared__ __align__(16) uint8_t tA[2][BM * PT];   // FP6 operand tails
  __shared__ __align__(16) uint8_t tW[2][BN * PT];
  __shared__ __align__(16) float sSA[2][2][BM];   // [stage][64-k half][row]
  __shared__ __align__(16) float sSW[2][2][BN];
  // scale stores of the threads past the tile's BM + BN scale rows (TM = 256:
  // waves 6, 7), never read: a destination for them keeps the staging store
  // branch-free (a branch in the pipelined stage made the compiler spill
  // ~1 KB per lane)
  constexpr int kSpare = kThreads - BM - BN;
  __shared__ __align__(16) float sSX[2][2][kSpare > 0 ? kSpare : 1];

  // ---- tile raster: XCD-contiguous ranges, then groups of kGroupRows tile-rows;
  // with a K split, workgroup b takes K range b / tiles of tile b % tiles
  const int nblk = p.tiles_m * p.tiles_n;
  const int split = blockIdx.x / nblk;
  int bid = blockIdx.x - split * nblk;
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
  // this workgroup's K stages [kb, ke) (whole groups: the host splits on group
  // boundaries)
  const int kb = split * p.stages_per_split;
  const int ke = min(p.K / BK, kb + p.stages_per_split);

  // ---- staging: each thread fetches 2 x 16 B of A (rows r, r + HALF) and
  // 16 B of W (row r; TM = 128: also r + 64) per stage through
  // buffer resources over the tile's rows (the host keeps a tile's rows
  // < 2^31 bytes), the stage's k offset in the scalar offset
  const int a_rows = min(BM, p.M - tile_m), w_rows = min(BN, p.N - tile_n);
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(p.a + (int64_t)tile_m * row_bytes, a_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(p.w + (int64_t)tile_n * row_bytes, w_rows * row_bytes);
  const int vA0 = min(tid >> 2, a_rows - 1) * row_bytes + (tid & 3) * 16;
  const int vA1 = min(HALF + (tid >> 2), a_rows - 1) * row_bytes + (tid & 3) * 16;
  const int vW0 = min(tid >> 2, w_rows - 1) * row_bytes + (tid & 3) * 16;
  const int vW1 = min(64 + (tid >> 2), w_rows - 1) * row_bytes + (tid & 3) * 16;
  const int st0 = main_off(tid >> 2, tid & 3);      // chunk tid & 3 of row tid >> 2
  const int st1 = st0 + HALF * PM;                   // row + HALF: same swizzle
  const int tt0 = tail_off(tid >> 2, tid & 3);
  const int tt1 = tt0 + HALF * PT;
  // scales: threads [0, BM) stage A-row scales, [BM, BM + 128) W-row scales
  // and any rest (TM = 256: waves 6, 7) a repeat of the last W row into a
  // dummy array;
  // group-major, so consecutive threads read consecutive rows of one group.
  // The choice is uniform per wave, so each wave's resource is scalar.
  const bool s_is_a = __builtin_amdgcn_readfirstlane(tid) < BM;
  const int srow = s_is_a ? tid : tid - BM;
  const float* sbase = s_is_a ? p.sa + tile_m : p.sw + tile_n;   // this tile's rows of group 0
  const int64_t sgs = s_is_a ? p.M : p.N;                      // floats between groups
  const int snr = s_is_a ? a_rows : w_rows;
  const int vS = 4 * min(srow, snr - 1);
  const int ssh = s_is_a ? p.sha : p.shw;
  float* sS = s_is_a ? &sSA[0][0][srow] : (kSpare <= 0 || srow < BN) ? &sSW[0][0][srow] : &sSX[0][0][srow - BN];
  const int sstr = s_is_a ? BM : BN;          // floats between the [half] rows of this thread's array

  // Two register sets of staged global data: stage kt+2 is fetched while
  // stage kt is computed and stage kt+1 (fetched one stage earlier) is
  // unpacked into LDS, so every load has two stages to land. The g = 64 mode
  // keeps one set (one stage ahead) to stay in registers. The partials export
  // runs each mode's schedule unchanged (same loads, ring depth and pipeline).
  constexpr int kAhead = (MODE == G64) ? 1 : 2;
  // scale of group column c for the thread's row: a per-stage scalar resource
  auto load_scale = [&](int c) -> float {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(sbase + c * sgs, 4 * snr);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vS, 0, 0));
  };
  struct Staged {
    uint4 a0, a1, w0, w1;
    float s0, s1;
  };
#define GLOAD(R, KT)                                                  \
  {                                                                   \
    const int off_ = (KT) * ROW_BYTES;                                \
    R.a0 = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rA, vA0, off_, 0)); \
    R.a1 = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rA, vA1, off_, 0)); \
    R.w0 = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rW, vW0, off_, 0)); \
    if constexpr (W2) R.w1 = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rW, vW1, off_, 0)); \
    R.s0 = load_scale((2 * (KT)) >> ssh);                             \
    /* groups >= 128: both 64-k halves share a group */               \
    R.s1 = (MODE == G64) ? load_scale((2 * (KT) + 1) >> ssh) : R.s0;  \
  }
// Staging stores of register set R into LDS buffer BUF, one piece at a time
// (the pipelined g = 128 stage spreads them over its chunks), or all at once.
#define LST_A0(BUF, R) unpack_store(&sA[BUF][st0], &tA[BUF][tt0], R.a0)
#define LST_A1(BUF, R) unpack_store(&sA[BUF][st1], &tA[BUF][tt1], R.a1)
#define LST_W0(BUF, R) unpack_store(&sW[BUF][st0], &tW[BUF][tt0], R.w0)
#define LST_W1(BUF, R) \
  if constexpr (W2) unpack_store(&sW[BUF][st1], &tW[BUF][tt1], R.w1)
#define LST_S(BUF, R)                                                 \
  {                                                                   \
    sS[(BUF) * 2 * sstr] = R.s0;                                      \
    sS[(BUF) * 2 * sstr + sstr] = R.s1;                               \
  }
#define LSTORE(BUF, R)                                                \
  {                                                                   \
    LST_A0(BUF, R);                                                   \
    LST_A1(BUF, R);                                                   \
    LST_W0(BUF, R);                                                   \
    LST_W1(BUF, R);                                                   \
    LST_S(BUF, R);                                                    \
  }

  const v16f zero16 = {};
  const v32f zero32 = {};
  v16f acc[2][2];
  v16f P[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = zero16;
      P[i][j] = zero16;
    }

  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  // lane operand: row (wm|wn)*64 + 32i + l32, chunk 2s + lhi; row + 32i has the
  // same swizzle as row, so one offset per k-step s serves both row blocks
  int rdA[2], rdW[2], rtA[2], rtW[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    rdA[s] = main_off(wm * 64 + l32, 2 * s + lhi);
    rdW[s] = main_off(wn * 64 + l32, 2 * s + lhi);
    rtA[s] = tail_off(wm * 64 + l32, 2 * s + lhi);
    rtW[s] = tail_off(wn * 64 + l32, 2 * s + lhi);
  }
  // G128 pipeline: scale product of tiles (0,1), (1,1) carried into the next
  // stage with their partials (zero before the first stage, so its carried
  // epilogue adds nothing)
  GroupScales Tc{zero32, 0.0f, 0.0f};
  int gcount = 0;     // GBIG: stages accumulated into P since the last epilogue
  int gidx = 0;       // index of the next group to finish (partials export)

  // Epilogue of tile (i, j) for group scales T (two-block product, block i).
#define EPI(I, J, T)                                                                     \
  {                                                                                      \
    if constexpr (PARTIALS) {                                                            \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                   \
        const int m = tile_m + wm * 64 + (I) * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);    \
        const int n = tile_n + wn * 64 + (J) * 32 + l32;                                 \
        if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)                \
          p.partials[((int64_t)gidx * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] =          \
              (int32_t)P[I][J][r];                                                       \
      }                                                                                  \
    } else if constexpr (ROWA) {                                                         \
      const float swj_ = (J) == 0 ? (T).sw0 : (T).sw1;                                   \
      _Pragma("unroll") for (int r = 0; r < 16; ++r)                                     \
        acc[I][J][r] = fmaf(P[I][J][r], swj_, acc[I][J][r]);                             \
    } else {                                                                             \
      _Pragma("unroll") for (int r = 0; r < 16; ++r)                                     \
        acc[I][J][r] = fmaf(P[I][J][r], (T).t[16 * (I) + r], acc[I][J][r]);              \
    }                                                                                    \
  }
  // End of a pipeline chunk: its MFMA issues first, then up to NV vector
  // instructions, then its LDS traffic; nothing crosses into the next chunk.
#define CHUNK_END(NV)                                                                    \
  {                                                                                      \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   \
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);                                  \
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);                                   \
    __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);                                   \
    __builtin_amdgcn_sched_barrier(0);                                                   \
  }
  // Half H (registers 8H .. 8H+7) of the epilogue of tile (I, J) for the group
  // with index GI; the partials export stores those registers instead (a
  // carried tile of the first stage, GI = -1, holds nothing).
#define EPI_HALF(I, J, T, H, GI)                                                         \
  {                                                                                      \
    if constexpr (PARTIALS) {                                                            \
      if ((GI) >= 0) {                                                                   \
        _Pragma("unroll") for (int r = 8 * (H); r < 8 * (H) + 8; ++r) {                  \
          const int m = tile_m + wm * 64 + (I) * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);  \
          const int n = tile_n + wn * 64 + (J) * 32 + l32;                               \
          if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)              \
            p.partials[((int64_t)(GI) * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] =        \
                (int32_t)P[I][J][r];                                                     \
        }                                                                                \
      }                                                                                  \
    } else if constexpr (ROWA) {                                                         \
      const float swj_ = (J) == 0 ? (T).sw0 : (T).sw1;                                   \
      _Pragma("unroll") for (int r = 8 * (H); r < 8 * (H) + 8; ++r)                      \
        acc[I][J][r] = fmaf(P[I][J][r], swj_, acc[I][J][r]);                             \
    } else {                                                                             \
      _Pragma("unroll") for (int r = 8 * (H); r < 8 * (H) + 8; ++r)                      \
        acc[I][J][r] = fmaf(P[I][J][r], (T).t[16 * (I) + r], acc[I][J][r]);              \
    }                                                                                    \
  }
  // Group scales for tiles (0, J) and (1, J) from scale values already read
  // (SA: the lane's A-row scale, SW: its W-column scale of column block J).
#define TPRODV(SA, SW, SW1)                                                              \
  GroupScales{ROWA ? zero32 : __builtin_amdgcn_mfma_f32_32x32x1f32(SA, SW, zero32, 0, 0, 0), \
              ROWA ? (SW) : 0.0f, ROWA ? (SW1) : 0.0f}
  // Group scales for tiles (0, J) and (1, J) from 64-k half H of stage buffer B:
  // the two-block product s_a x s_w, or (ROWA) the lane's two W scales.
#define TPROD(B, H, J)                                                                   \
  GroupScales{ROWA ? zero32 : __builtin_amdgcn_mfma_f32_32x32x1f32(                      \
                   sSA[B][H][wm * 64 + lane], sSW[B][H][wn * 64 + 32 * (J) + l32], zero32, 0, 0, 0), \
               ROWA ? sSW[B][H][wn * 64 + l32] : 0.0f,                                   \
               ROWA ? sSW[B][H][wn * 64 + 32 + l32] : 0.0f}

  // One K stage from LDS buffer BUF: fetch stage min(KT+kAhead, ke-1) into
  // register set RL, compute, unpack register set RS (stage KT+1) into buffer
  // BUF^1. The
  // fetch and the store are unconditional (at the end they repeat the final
  // stage into the idle buffer): a branch would let the compiler sink the MFMAs
  // below the store. Phase order is pinned with scheduling barriers: each
  // tile's epilogue is issued next to the following tile's MFMAs, the unpack
  // next to the last MFMAs, and the two scale-product blocks are never live
  // together.
#define STAGE(KT, BUF, RL, RS)                                                           \
  {                                                                                      \
    GLOAD(RL, min((KT) + kAhead, ke - 1));                                               \
    const uint8_t* bA = sA[BUF];                                                         \
    const uint8_t* bW = sW[BUF];                                                         \
    const uint8_t* cA = tA[BUF];                                                         \
    const uint8_t* cW = tW[BUF];                                                         \
    v8i a[2][2], b[2][2];   /* [tile row i / col j][k-step s] */                         \
    /* operands of k-step S; g = 64 reads each step's just before its MFMAs */          \
    /* (the barriers keep the compiler from merging two operands' 8-byte     */      \
    /* tails into one read, which would need register moves to split them)  */      \
    auto load_step = [&](int S) {                                                        \
      _Pragma("unroll") for (int i = 0; i < 2; ++i) {                                    \
        a[i][S] = load_op(bA + rdA[S] + i * 32 * PM, cA + rtA[S] + i * 32 * PT);         \
        __builtin_amdgcn_sched_barrier(0);                                               \
        b[i][S] = load_op(bW + rdW[S] + i * 32 * PM, cW + rtW[S] + i * 32 * PT);         \
        __builtin_amdgcn_sched_barrier(0);                                               \
      }                                                                                  \
    };                                                                                   \
    /* W operands of column block 1 (G128 pipeline: read mid-stage) */                \
    auto load_w1 = [&]() {                                                               \
      _Pragma("unroll") for (int S = 0; S < 2; ++S) {                                    \
        b[1][S] = load_op(bW + rdW[S] + 32 * PM, cW + rtW[S] + 32 * PT);                 \
        __builtin_amdgcn_sched_barrier(0);                                               \
      }                                                                                  \
    };                                                                                   \
    if constexpr (MODE == G128) {                                                        \
      a[0][0] = load_op(bA + rdA[0], cA + rtA[0]);                                       \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      b[0][0] = load_op(bW + rdW[0], cW + rtW[0]);                                       \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      a[1][0] = load_op(bA + rdA[0] + 32 * PM, cA + rtA[0] + 32 * PT);                   \
      __builtin_amdgcn_sched_barrier(0);                                                 \
    } else if constexpr (MODE != G64) {                                                  \
      load_step(0);                                                                      \
      load_step(1);                                                                      \
    }                                                                                    \
    if constexpr (MODE == G64) {                                                         \
      _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                    \
        /* one tile at a time (its MFMA, then its epilogue): with a group per    */   \
        /* k-step, keeping two tiles' partials in flight does not fit the VGPRs   */   \
        load_step(s);                                                                    \
        const GroupScales T0 = TPROD(BUF, s, 0);                                         \
        P[0][0] = mma(a[0][s], b[0][s], zero16);                                         \
        EPI(0, 0, T0);                                                                   \
        P[1][0] = mma(a[1][s], b[0][s], zero16);                                         \
        EPI(1, 0, T0);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                               \
        const GroupScales T1 = TPROD(BUF, s, 1);                                         \
        P[1][1] = mma(a[1][s], b[1][s], zero16);                                         \
        EPI(1, 1, T1);                                                                   \
        if (s == 1) LSTORE((BUF) ^ 1, RS);                                               \
        P[0][1] = mma(a[0][s], b[1][s], zero16);                                         \
        EPI(0, 1, T1);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                               \
        ++gidx;                                                                          \
      }                                                                                  \
    } else if constexpr (MODE == G128) {                                                 \
      /* Software pipeline: ten chunks, each one MFMA issued first and the     */    \
      /* vector work that runs under it. An epilogue reads partials finished  */    \
      /* two MFMAs or more earlier (no dependency wait); tiles (1,1) and      */    \
      /* (0,1) are finished under the next stage's first four MFMAs (their    */    \
      /* partials and scale product Tc carried over). Tc dies before T0 is    */    \
      /* formed and T0 before the next Tc, so one scale product is live.      */    \
      /* the stage's scale values (tile rows / columns of this lane) */                 \
      const float gsa_ = sSA[BUF][0][wm * 64 + lane];                                    \
      const float gsw0_ = sSW[BUF][0][wn * 64 + l32];                                    \
      const float gsw1_ = sSW[BUF][0][wn * 64 + 32 + l32];                               \
      P[0][0] = mma(a[0][0], b[0][0], zero16);                                           \
      EPI_HALF(1, 1, Tc, 0, gidx - 1);                                                   \
      a[0][1] = load_op(bA + rdA[1], cA + rtA[1]);                                       \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      b[0][1] = load_op(bW + rdW[1], cW + rtW[1]);                                       \
      CHUNK_END(8);                                                                      \
      P[1][0] = mma(a[1][0], b[0][0], zero16);                                           \
      EPI_HALF(1, 1, Tc, 1, gidx - 1);                                                   \
      LST_A0((BUF) ^ 1, RS);                                                             \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      a[1][1] = load_op(bA + rdA[1] + 32 * PM, cA + rtA[1] + 32 * PT);                   \
      CHUNK_END(16);                                                                     \
      P[0][0] = mma(a[0][1], b[0][1], P[0][0]);                                          \
      EPI_HALF(0, 1, Tc, 0, gidx - 1);                                                   \
      CHUNK_END(8);                                                                      \
      P[1][0] = mma(a[1][1], b[0][1], P[1][0]);                                          \
      EPI_HALF(0, 1, Tc, 1, gidx - 1);                                                   \
      LST_A1((BUF) ^ 1, RS);                                                             \
      CHUNK_END(16);                                                                     \
      GroupScales T0 = TPRODV(gsa_, gsw0_, gsw1_);                                       \
      if constexpr (!ROWA) asm volatile("" : "+v"(T0.t));   /* no product with per-token A scales */ \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      load_w1();                                                                         \
      CHUNK_END(16);                                                                     \
      P[1][1] = mma(a[1][0], b[1][0], zero16);                                           \
      EPI_HALF(0, 0, T0, 0, gidx);                                                       \
      CHUNK_END(8);                                                                      \
      P[0][1] = mma(a[0][0], b[1][0], zero16);                                           \
      EPI_HALF(0, 0, T0, 1, gidx);                                                       \
      LST_W0((BUF) ^ 1, RS);                                                             \
      CHUNK_END(16);                                                                     \
      P[1][1] = mma(a[1][1], b[1][1], P[1][1]);                                          \
      EPI_HALF(1, 0, T0, 0, gidx);                                                       \
      CHUNK_END(8);                                                                      \
      P[0][1] = mma(a[0][1], b[1][1], P[0][1]);                                          \
      EPI_HALF(1, 0, T0, 1, gidx);                                                       \
      LST_W1((BUF) ^ 1, RS);                                                             \
      CHUNK_END(16);                                                                     \
      Tc = TPRODV(gsa_, gsw1_, gsw1_);                                                   \
      LST_S((BUF) ^ 1, RS);                                                              \
      CHUNK_END(16);                                                                     \
      /* keep Tc's MFMA here (it would sink into the next stage) */                     \
      if constexpr (!ROWA) asm volatile("" : "+v"(Tc.t));   /* no product with per-token A scales */ \
      ++gidx;                                                                            \
    } else {                                                                             \
      /* partials accumulate over stages_per_group stages, then one epilogue */          \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                      \
      _Pragma("unroll") for (int j = 0; j < 2; ++j)                                      \
        P[i][j] = mma(a[i][1], b[j][1], mma(a[i][0], b[j][0], P[i][j]));                 \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      LSTORE((BUF) ^ 1, RS);                                                             \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      if (++gcount == p.stages_per_group) {                                              \
        const GroupScales T0 = TPROD(BUF, 0, 0);                                         \
        EPI(0, 0, T0);                                                                   \
        EPI(1, 0, T0);                                                                   \
        const GroupScales T1 = TPROD(BUF, 0, 1);                                         \
        EPI(0, 1, T1);                                                                   \
        EPI(1, 1, T1);                                                                   \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                    \
        _Pragma("unroll") for (int j = 0; j < 2; ++j) P[i][j] = zero16;                  \
        gcount = 0;                                                                      \
        ++gidx;                                                                          \
      }                                                                                  \
    }                                                                                    \
    lds_barrier();                                                                       \
  }

  Staged R0, R1;
  Staged& RX = (kAhead == 2) ? R1 : R0;
  GLOAD(R0, kb);
  LSTORE(0, R0);
  if constexpr (kAhead == 2) GLOAD(R1, min(kb + 1, ke - 1));
  lds_barrier();
  int kt = kb;
  for (; kt + 1 < ke; kt += 2) {
    STAGE(kt, 0, R0, RX);
    STAGE(kt + 1, 1, RX, R0);
  }
  if (kt < ke) STAGE(kt, 0, R0, RX);
  if constexpr (MODE == G128) {   // the last stage's carried tiles
    EPI_HALF(1, 1, Tc, 0, gidx - 1);
    EPI_HALF(1, 1, Tc, 1, gidx - 1);
    EPI_HALF(0, 1, Tc, 0, gidx - 1);
    EPI_HALF(0, 1, Tc, 1, gidx - 1);
  }
#undef GLOAD
#undef LSTORE
#undef LST_A0
#undef LST_A1
#undef LST_W0
#undef LST_W1
#undef LST_S
#undef EPI_HALF
#undef CHUNK_END
#undef EPI
#undef TPROD
#undef TPRODV
#undef STAGE

  if constexpr (!PARTIALS) {
    const int esz = p.ydtype == 0 ? 4 : 2;
    void* const yb = static_cast<uint8_t*>(p.y) + split * p.split_stride * esz;   // this split's output
    if (tile_m + BM <= p.M && (int64_t)BM * p.ldy * esz < (int64_t{1} << 31)) {
      // Every row of the tile is valid and the tile spans < 2^31 bytes: buffer
      // stores with each register's row offset in the scalar offset, no
      // per-element address arithmetic or branches. A lane whose column is
      // >= N gets an offset past the resource, so its stores are dropped.
      const int ldb = (int)(p.ldy * esz);
      const __amdgpu_buffer_rsrc_t rY =
          buffer_rsrc(static_cast<uint8_t*>(yb) + (int64_t)tile_m * ldb, BM * ldb);
      const int row0 = wm * 64 + 4 * lhi;                // tile row of register 0, block 0
      int voffY[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = tile_n + wn * 64 + j * 32 + l32;
        voffY[j] = n < p.N ? row0 * ldb + n * esz : kDroppedOffset;
      }
      const float* sa_rows = p.sa + tile_m + row0;       // ROWA: xs[m], one group
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dr = i * 32 + 8 * (r >> 2) + (r & 3);
          const int soff = dr * ldb;
          const float sa = ROWA ? sa_rows[dr] : 1.0f;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float v = ROWA ? acc[i][j][r] * sa : acc[i][j][r];
            if (p.ydtype == 0)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rY, voffY[j], soff, kStoreNT);
            else
              __builtin_amdgcn_raw_buffer_store_b16(__half_as_ushort(__float2half_rn(v)), rY, voffY[j], soff, kStoreNT);
          }
        }
    } else {
      // last row tile of a ragged M (or a huge ldy): per-element checked stores
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = tile_m + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
            const int n = tile_n + wn * 64 + j * 32 + l32;
            if (m < p.M && n < p.N) {
              const float v = ROWA ? acc[i][j][r] * p.sa[m] : acc[i][j][r];   // one group: xs[m]
              if (p.ydtype == 0)
                static_cast<float*>(yb)[(int64_t)m * p.ldy + n] = v;
              else
                static_cast<__half*>(yb)[(int64_t)m * p.ldy + n] = __float2half_rn(v);
            }
          }
    }
  }
}

// Sum of the K splits' fp32 outputs ws[s][M][N] in split order (deterministic),
// stored as fp32 or fp16 into y[M][ldy]. Each thread takes four consecutive
// columns of a row (N % 4 == 0) or one element.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int splits, int M, int N,
                                                      int64_t split_stride, void* __restrict__ y, int ydtype,
                                                      int64_t ldy) {
  const int vec = (N & 3) == 0 ? 4 : 1;
  const int64_t per_row = N / vec, total = (int64_t)M * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / per_row;
    const int n = (int)(i - m * per_row) * vec;
    const float* src = ws + m * N + n;
    if (vec == 4) {
      float4 a = *reinterpret_cast<const float4*>(src);
      for (int s = 1; s < splits; ++s) {
        const float4 b = *reinterpret_cast<const float4*>(src + s * split_stride);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
      }
      if (ydtype == 0) {
        float* d = static_cast<float*>(y) + m * ldy + n;
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
      } else {
        __half* d = static_cast<__half*>(y) + m * ldy + n;
        d[0] = __float2half_rn(a.x); d[1] = __float2half_rn(a.y);
        d[2] = __float2half_rn(a.z); d[3] = __float2half_rn(a.w);
      }
    } else {
      float a = src[0];
      for (int s = 1; s < splits; ++s) a += src[s * split_stride];
      if (ydtype == 0)
        static_cast<float*>(y)[m * ldy + n] = a;
      else
        static_cast<__half*>(y)[m * ldy + n] = __float2half_rn(a);
    }
  }
}

// ---- Small M (decode) ------------------------------------------------------
// With few tokens the big tiling leaves most CUs idle (LLaMA-2-70B w2 at
// M = 1: 64 tiles for 256 CUs, each walking all of K) and the GEMM is bound by
// streaming W. This path gives each workgroup one 32 x 32 output tile (one
// MFMA block) and splits K between its NW waves in whole groups: wave w
// takes groups [G w / NW, G (w + 1) / NW). Eight waves when the launch has
// fewer than 512 workgroups (more loads in flight per CU), else four. Operands go straight from memory into
// registers (W is read once, A stays in L2) through an 8-step ring of loads in
// flight, are widened there, and run through the same FP6 MFMA, partials and
// epilogue arithmetic as the tiled kernel. The four waves' accumulators are
// summed through LDS in a fixed order (wave 0, then 1, 2, ...): deterministic.
constexpr int SM_TILE = 32;

constexpr int SM_RING = 8;          // 64-k steps in flight per wave (a multiple of 4)
static_assert(SM_RING % 4 == 0, "the ring is refilled four steps at a time");

// 32 packed codes (16 B = two units X0 Y0 X1 Y1) -> the lane's FP6 operand in
// registers: the words unpack_store() writes to LDS, main part then tail.
__device__ __forceinline__ v8i widen(uint4 v) {
  const v4i lo = v4i{(int)(v.x & ~kFoldX), (int)((v.x & kFoldX) | (v.y & kFoldY)),
                     (int)(v.y & ~kFoldY), (int)(v.z & ~kFoldX)};
  const v4i hi = v4i{(int)((v.z & kFoldX) | (v.w & kFoldY)), (int)(v.w & ~kFoldY), 0, 0};
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, -1, -1);
}

template <bool PARTIALS, bool ROWA, int SM_WAVES>
__global__ __launch_bounds__(64 * SM_WAVES) void k_w4a4_gemm_small(Params p, int steps_per_group) {
  __shared__ float red[SM_WAVES - 1][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;
  const int tile_m = (p.tile_m0 + (int)blockIdx.x % p.tiles_m) * SM_TILE;
  const int tile_n = (p.tile_n0 + (int)blockIdx.x / p.tiles_m) * SM_TILE;
  const int row_bytes = p.K >> 1;
  const int a_rows = min(SM_TILE, p.M - tile_m), w_rows = min(SM_TILE, p.N - tile_n);
  // rows past the matrix lie past the resources and read as zero codes / scales
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(p.a + (int64_t)tile_m * row_bytes, a_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(p.w + (int64_t)tile_n * row_bytes, w_rows * row_bytes);
  const int voff = l32 * row_bytes + 16 * lhi;        // row l32, 32-code chunk lhi of a 64-k step
  const int groups = p.K / (64 * steps_per_group);
  const int h0 = groups * wave / SM_WAVES * steps_per_group;
  const int h1 = groups * (wave + 1) / SM_WAVES * steps_per_group;

  struct Step {
    uint4 a, w;
    float sa, sw;
  };
  // operands of 64-k step h and the scales of its group's column
  auto load = [&](Step& st, int h) {
    st.a = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rA, voff, h * 32, 0));
    st.w = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rW, voff, h * 32, 0));
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.sa + (int64_t)(h >> p.sha) * p.M + tile_m, 4 * a_rows);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.sw + (int64_t)(h >> p.shw) * p.N + tile_n, 4 * w_rows);
    st.sa = ROWA ? 0.0f : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, 4 * l32, 0, 0));
    st.sw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, 4 * l32, 0, 0));
  };

  const v16f zero16 = {};
  const v32f zero32 = {};
  v16f acc = zero16, P = zero16;
  int in_group = 0;
  Step ring[SM_RING];
#pragma unroll
  for (int u = 0; u < SM_RING; ++u)
    if (h0 + u < h1) load(ring[u], h0 + u);
  for (int h = h0; h < h1; h += SM_RING) {
#pragma unroll
    for (int u = 0; u < SM_RING; ++u) {
      if (h + u < h1) {
        P = mma(widen(ring[u].a), widen(ring[u].w), P);
        if (++in_group == steps_per_group) {
          in_group = 0;
          if constexpr (PARTIALS) {
            const int gidx = (h + u) / steps_per_group;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = tile_m + 8 * (r >> 2) + 4 * lhi + (r & 3);
              const int n = tile_n + l32;
              if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)
                p.partials[((int64_t)gidx * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] = (int32_t)P[r];
            }
          } else if constexpr (ROWA) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf(P[r], ring[u].sw, acc[r]);
          } else {
            // s_a x s_w for the tile: block 0 of the two-block rank-1 product
            const v32f t = __builtin_amdgcn_mfma_f32_32x32x1f32(ring[u].sa, ring[u].sw, zero32, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = fmaf(P[r], t[r], acc[r]);
          }
          P = zero16;
        }
      }
      // refill four steps at once: a row's four 32-byte pieces of one 128-byte
      // W line go out back to back (one per step refilled one at a time
      // streamed W 7-19 % slower at M = 1)
      if ((u & 3) == 3) {
#pragma unroll
        for (int v = u - 3; v <= u; ++v)
          if (h + SM_RING + v < h1) load(ring[v], h + SM_RING + v);
      }
    }
  }
  if constexpr (!PARTIALS) {
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave - 1][r][lane] = acc[r];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < SM_WAVES - 1; ++w)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += red[w][r][lane];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = tile_m + 8 * (r >> 2) + 4 * lhi + (r & 3);
        const int n = tile_n + l32;
        if (m < p.M && n < p.N) {
          const float v = ROWA ? acc[r] * p.sa[m] : acc[r];   // one group: xs[m]
          if (p.ydtype == 0)
            static_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = v;
          else
            static_cast<__half*>(p.y)[(int64_t)m * p.ldy + n] = __float2half_rn(v);
        }
      }
    }
  }
}

// ---- Few tokens, 16-column tiles ----------------------------------------------
// For M <= 16 and groups of 128 or more: one 16 x 16 output tile per workgroup
// on the 16x16x128 FP6 instruction. Its operand lane layout (row l % 16,
// 32-code chunk l / 16 of a 128-k step) makes each load instruction read 64
// contiguous bytes from each of 16 W rows, where the 32 x 32 tile reads 32
// bytes from each of 32 rows: measured on a W stream of the LLaMA-2-70B w1
// shape, 6.5 against 5.35 TB/s. Twice as many workgroups also spread evenly
// over the CUs where the 32-column grid does not (896 = 3.5 per CU for
// N = 28672). Same K split between the waves (whole groups), same exact
// integer partials and epilogue order as k_w4a4_gemm_small, so Y is
// bit-identical to it; the scale product is one multiply per output.
constexpr int SM16_TILE = 16;
// 128-k steps in flight per wave, refilled two at a time. A short ring keeps the
// kernel at ~52 VGPRs, so every workgroup of a LLaMA-2-70B w1 launch (1792)
// is resident at once; rings of 4 and 8 (78 / 130 VGPRs: 1536 / 768 resident
// workgroups) measured slower at M = 1, 4 and 16 with W streamed from HBM
// (w1 M = 4: 30.0 / 30.3 / 33.5 us).
constexpr int SM16_RING = 2;

typedef float v4f_16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f_16 mma16(const v8i& a, const v8i& b, const v4f_16& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp6, kFmtFp6, 0, kUnitScale, 0, kUnitScale);
}

template <bool PARTIALS, int SM_WAVES>
__global__ __launch_bounds__(64 * SM_WAVES) void k_w4a4_gemm_small16(Params p, int steps_per_group) {
  __shared__ float red[SM_WAVES - 1][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int tile_m = (p.tile_m0 + (int)blockIdx.x % p.tiles_m) * SM16_TILE;
  const int tile_n = (p.tile_n0 + (int)blockIdx.x / p.tiles_m) * SM16_TILE;
  const int row_bytes = p.K >> 1;
  const int a_rows = min(SM16_TILE, p.M - tile_m), w_rows = min(SM16_TILE, p.N - tile_n);
  // rows past the matrix lie past the resources and read as zero codes / scales
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(p.a + (int64_t)tile_m * row_bytes, a_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(p.w + (int64_t)tile_n * row_bytes, w_rows * row_bytes);
  const int voff = l16 * row_bytes + 16 * lq;         // row l16, 32-code chunk lq of a 128-k step
  const int groups = p.K / (128 * steps_per_group);
  const int h0 = groups * wave / SM_WAVES * steps_per_group;
  const int h1 = groups * (wave + 1) / SM_WAVES * steps_per_group;

  struct Step {
    uint4 a, w;
    float4 sa;   // the scales of the lane's four output rows 4 lq .. 4 lq + 3
    float sw;    // the scale of its output column l16
  };
  // operands of 128-k step h and the scales of its group's column
  auto load = [&](Step& st, int h) {
    st.a = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rA, voff, h * 64, 0));
    st.w = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rW, voff, h * 64, 0));
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.sa + (int64_t)((2 * h) >> p.sha) * p.M + tile_m, 4 * a_rows);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.sw + (int64_t)((2 * h) >> p.shw) * p.N + tile_n, 4 * w_rows);
    const v4u s4 = __builtin_amdgcn_raw_buffer_load_b128(ra, 16 * lq, 0, 0);
    st.sa = float4{__uint_as_float(s4.x), __uint_as_float(s4.y), __uint_as_float(s4.z), __uint_as_float(s4.w)};
    st.sw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, 4 * l16, 0, 0));
  };

  const v4f_16 zero4 = {};
  v4f_16 acc = zero4, P = zero4;
  int in_group = 0;
  Step ring[SM16_RING];
#pragma unroll
  for (int u = 0; u < SM16_RING; ++u)
    if (h0 + u < h1) load(ring[u], h0 + u);
  for (int h = h0; h < h1; h += SM16_RING) {
#pragma unroll
    for (int u = 0; u < SM16_RING; ++u) {
      if (h + u < h1) {
        P = mma16(widen(ring[u].a), widen(ring[u].w), P);
        if (++in_group == steps_per_group) {
          in_group = 0;
          if constexpr (PARTIALS) {
            const int gidx = (h + u) / steps_per_group;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = tile_m + 4 * lq + i;
              const int n = tile_n + l16;
              if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)
                p.partials[((int64_t)gidx * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] = (int32_t)P[i];
            }
          } else {
            const float sa[4] = {ring[u].sa.x, ring[u].sa.y, ring[u].sa.z, ring[u].sa.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fmaf(P[i], sa[i] * ring[u].sw, acc[i]);
          }
          P = zero4;
        }
      }
      // refill two steps at once: a row's two 64-byte pieces of one 128-byte
      // W line go out back to back
      if ((u & 1) == 1) {
#pragma unroll
        for (int v = u - 1; v <= u; ++v)
          if (h + SM16_RING + v < h1) load(ring[v], h + SM16_RING + v);
      }
    }
  }
  if constexpr (!PARTIALS) {
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < SM_WAVES - 1; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += red[w][i][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = tile_m + 4 * lq + i;
        const int n = tile_n + l16;
        if (m < p.M && n < p.N) {
          if (p.ydtype == 0)
            static_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = acc[i];
          else
            static_cast<__half*>(p.y)[(int64_t)m * p.ldy + n] = __float2half_rn(acc[i]);
        }
      }
    }
  }
}

// ---- Few tokens, activations quantized in the GEMM (fused decode path) -------
// At decode the activation quantization is a launch of its own in front of a
// ~25-35 us W stream. Here each workgroup quantizes all M x K activations
// itself -- dense lanes, one 32-element chunk per lane, the quantizer's
// arithmetic (quant_common.h) -- into an LDS copy of their FP6 operand stream
// and scales, then runs the few-token loop above with A operands read from
// LDS. Every workgroup repeats the quantization (M x K elements), so the path
// pays only for tiny M x K; its W loads are issued before the quantization so
// the stream starts at once. Codes, scales, partials and the epilogue are the
// quantizer's and k_w4a4_gemm_small's: Y is bit-identical to w4a4_quantize_act
// followed by w4a4_gemm.
struct LinParams {
  const uint16_t* x;
  int64_t ldx;
  const uint8_t* w;
  const float* sw;
  int sha, shw;               // scale column of 64-k step h = h >> sh
  int M, N, K;
  void* y;
  int ydtype;
  int64_t ldy;
};

// The fused kernels' prologue: every 32-element chunk of X quantized into
// the workgroup's LDS copy (FP6 operand words 0..3 in qm, 4..5 in qt, one
// scale per group in ss) by NT threads, one chunk per thread per pass. A
// version that fetched the next pass's chunk during this one measured no
// faster at M = 1..4: the prologue's cost is its M x K re-read per workgroup.
template <int LPG, int NT>
__device__ __forceinline__ void quantize_to_lds(const LinParams& p, int cpr, int gpr, uint4* qm, uint2* qt,
                                                float* ss) {
  const float nz = opaque_neg_zero();
  const int total = p.M * cpr;                  // a multiple of LPG: groups stay whole
  for (int c = threadIdx.x; c < total; c += NT) {
    const int row = c / cpr, col = c - row * cpr;
    const uint4* src = reinterpret_cast<const uint4*>(p.x + row * p.ldx + col * 32);
    uint4 raw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = src[j];
    uint32_t wd[16];
    words16(raw, wd);
    const float a = group_max<LPG>(absmax_words<16>(wd));
    float sc, r8, s8;
    group_scale(a, sc, r8, s8);
    const v6u f = int4_stream<16>(wd, r8, s8, nz);
    qm[c] = uint4{f[0], f[1], f[2], f[3]};
    qt[c] = uint2{f[4], f[5]};
    if (col % LPG == 0) ss[row * gpr + col / LPG] = sc;
  }
}

template <int G, int SM_WAVES>
__global__ __launch_bounds__(64 * SM_WAVES) void k_w4a4_linear_small(LinParams p, int steps_per_group) {
  constexpr int LPG = G / 32;                   // lanes (32-element chunks) per activation group
  extern __shared__ __align__(16) uint8_t lds[];
  const int cpr = p.K >> 5;                     // chunks per row
  const int gpr = p.K / G;                      // activation groups per row
  uint4* qm = reinterpret_cast<uint4*>(lds);                          // [M][cpr] operand words 0..3
  uint2* qt = reinterpret_cast<uint2*>(lds + 16 * p.M * cpr);         // [M][cpr] operand words 4, 5
  float* ss = reinterpret_cast<float*>(lds + 24 * p.M * cpr);         // [M][gpr] scales
  float* red = ss + p.M * gpr;                                        // [SM_WAVES - 1][16][64]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;
  const int tile_n = (int)blockIdx.x * SM_TILE;
  const int row_bytes = p.K >> 1;
  const int w_rows = min(SM_TILE, p.N - tile_n);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(p.w + (int64_t)tile_n * row_bytes, w_rows * row_bytes);
  const int voff = l32 * row_bytes + 16 * lhi;
  const int groups = p.K / (64 * steps_per_group);
  const int h0 = groups * wave / SM_WAVES * steps_per_group;
  const int h1 = groups * (wave + 1) / SM_WAVES * steps_per_group;

  struct Step {
    uint4 w;
    float sw;
  };
  auto load = [&](Step& st, int h) {
    st.w = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rW, voff, h * 32, 0));
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.sw + (int64_t)(h >> p.shw) * p.N + tile_n, 4 * w_rows);
    st.sw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, 4 * l32, 0, 0));
  };
  Step ring[SM_RING];
#pragma unroll
  for (int u = 0; u < SM_RING; ++u)
    if (h0 + u < h1) load(ring[u], h0 + u);

  // ---- prologue: the workgroup's copy of the quantized activations
  quantize_to_lds<LPG, 64 * SM_WAVES>(p, cpr, gpr, qm, qt, ss);
  __syncthreads();

  const bool arow = l32 < p.M;                  // the lane's A row exists
  const int abase = l32 * cpr + lhi;            // chunk of step h: abase + 2 h
  const v16f zero16 = {};
  const v32f zero32 = {};
  v16f acc = zero16, P = zero16;
  int in_group = 0;
  for (int h = h0; h < h1; h += SM_RING) {
#pragma unroll
    for (int u = 0; u < SM_RING; ++u) {
      if (h + u < h1) {
        v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
        if (arow) {
          const uint4 m4 = qm[abase + 2 * (h + u)];
          const uint2 t2 = qt[abase + 2 * (h + u)];
          a = v8i{(int)m4.x, (int)m4.y, (int)m4.z, (int)m4.w, (int)t2.x, (int)t2.y, 0, 0};
        }
        P = mma(a, widen(ring[u].w), P);
        if (++in_group == steps_per_group) {
          in_group = 0;
          const float sa = arow ? ss[l32 * gpr + ((h + u) >> p.sha)] : 0.0f;
          // s_a x s_w for the tile: block 0 of the two-block rank-1 product
          const v32f t = __builtin_amdgcn_mfma_f32_32x32x1f32(sa, ring[u].sw, zero32, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = fmaf(P[r], t[r], acc[r]);
          P = zero16;
        }
      }
      if ((u & 3) == 3) {
#pragma unroll
        for (int v = u - 3; v <= u; ++v)
          if (h + SM_RING + v < h1) load(ring[v], h + SM_RING + v);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave - 1) * 16 + r) * 64 + lane] = acc[r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < SM_WAVES - 1; ++w)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += red[(w * 16 + r) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * lhi + (r & 3);
      const int n = tile_n + l32;
      if (m < p.M && n < p.N) {
        if (p.ydtype == 0)
          static_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = acc[r];
        else
          static_cast<__half*>(p.y)[(int64_t)m * p.ldy + n] = __float2half_rn(acc[r]);
      }
    }
  }
}

// The fused path on 16-column tiles: the quantization prologue and LDS copy
// of k_w4a4_linear_small, the loads, instruction and epilogue of
// k_w4a4_gemm_small16 (A operands from the LDS copy: lane row l % 16, chunk
// 4 h + l / 16 of 128-k step h). Bit-identical to w4a4_quantize_act followed
// by w4a4_gemm on the same tiles.
template <int G, int SM_WAVES>
__global__ __launch_bounds__(64 * SM_WAVES) void k_w4a4_linear_small16(LinParams p, int steps_per_group) {
  constexpr int LPG = G / 32;                   // lanes (32-element chunks) per activation group
  extern __shared__ __align__(16) uint8_t lds[];
  const int cpr = p.K >> 5;                     // chunks per row
  const int gpr = p.K / G;                      // activation groups per row
  uint4* qm = reinterpret_cast<uint4*>(lds);                          // [M][cpr] operand words 0..3
  uint2* qt = reinterpret_cast<uint2*>(lds + 16 * p.M * cpr);         // [M][cpr] operand words 4, 5
  float* ss = reinterpret_cast<float*>(lds + 24 * p.M * cpr);         // [M][gpr] scales
  float* red = ss + p.M * gpr;                                        // [SM_WAVES - 1][4][64]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int tile_n = (int)blockIdx.x * SM16_TILE;
  const int row_bytes = p.K >> 1;
  const int w_rows = min(SM16_TILE, p.N - tile_n);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(p.w + (int64_t)tile_n * row_bytes, w_rows * row_bytes);
  const int voff = l16 * row_bytes + 16 * lq;
  const int groups = p.K / (128 * steps_per_group);
  const int h0 = groups * wave / SM_WAVES * steps_per_group;
  const int h1 = groups * (wave + 1) / SM_WAVES * steps_per_group;

  struct Step {
    uint4 w;
    float sw;
  };
  auto load = [&](Step& st, int h) {
    st.w = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rW, voff, h * 64, 0));
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.sw + (int64_t)((2 * h) >> p.shw) * p.N + tile_n, 4 * w_rows);
    st.sw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, 4 * l16, 0, 0));
  };
  Step ring[SM16_RING];
#pragma unroll
  for (int u = 0; u < SM16_RING; ++u)
    if (h0 + u < h1) load(ring[u], h0 + u);

  // ---- prologue: the workgroup's copy of the quantized activations
  quantize_to_lds<LPG, 64 * SM_WAVES>(p, cpr, gpr, qm, qt, ss);
  __syncthreads();

  const bool arow = l16 < p.M;                  // the lane's A row exists
  const int abase = l16 * cpr + lq;             // chunk of step h: abase + 4 h
  const v4f_16 zero4 = {};
  v4f_16 acc = zero4, P = zero4;
  int in_group = 0;
  for (int h = h0; h < h1; h += SM16_RING) {
#pragma unroll
    for (int u = 0; u < SM16_RING; ++u) {
      if (h + u < h1) {
        v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
        if (arow) {
          const uint4 m4 = qm[abase + 4 * (h + u)];
          const uint2 t2 = qt[abase + 4 * (h + u)];
          a = v8i{(int)m4.x, (int)m4.y, (int)m4.z, (int)m4.w, (int)t2.x, (int)t2.y, 0, 0};
        }
        P = mma16(a, widen(ring[u].w), P);
        if (++in_group == steps_per_group) {
          in_group = 0;
          const int gcol = (2 * (h + u)) >> p.sha;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 4 * lq + i;
            const float sa = m < p.M ? ss[m * gpr + gcol] : 0.0f;
            acc[i] = fmaf(P[i], sa * ring[u].sw, acc[i]);
          }
          P = zero4;
        }
      }
      if ((u & 1) == 1) {
#pragma unroll
        for (int v = u - 1; v <= u; ++v)
          if (h + SM16_RING + v < h1) load(ring[v], h + SM16_RING + v);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave - 1) * 4 + i) * 64 + lane] = acc[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < SM_WAVES - 1; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += red[(w * 4 + i) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * lq + i;
      const int n = tile_n + l16;
      if (m < p.M && n < p.N) {
        if (p.ydtype == 0)
          static_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = acc[i];
        else
          static_cast<__half*>(p.y)[(int64_t)m * p.ldy + n] = __float2half_rn(acc[i]);
      }
    }
  }
}

template <int NW>
void launch_small(const GemmArgs& g, const Params& p, dim3 grid, int spg, hipStream_t stream) {
  if (g.partials)
    hipLaunchKernelGGL((k_w4a4_gemm_small<true, false, NW>), grid, dim3(64 * NW), 0, stream, p, spg);
  else if (g.ga == g.K)
    hipLaunchKernelGGL((k_w4a4_gemm_small<false, true, NW>), grid, dim3(64 * NW), 0, stream, p, spg);
  else
    hipLaunchKernelGGL((k_w4a4_gemm_small<false, false, NW>), grid, dim3(64 * NW), 0, stream, p, spg);
}

template <int NW>
void launch_small16(const GemmArgs& g, const Params& p, dim3 grid, int spg, hipStream_t stream) {
  if (g.partials)
    hipLaunchKernelGGL((k_w4a4_gemm_small16<true, NW>), grid, dim3(64 * NW), 0, stream, p, spg);
  else
    hipLaunchKernelGGL((k_w4a4_gemm_small16<false, NW>), grid, dim3(64 * NW), 0, stream, p, spg);
}

// log2(group / 64) for a power-of-two group, 31 (a single column) for group == K.
int scale_shift(int64_t group, int64_t K) {
  if (group == K && (group & (group - 1))) return 31;
  int s = 0;
  while ((64LL << s) < group) ++s;
  return s;
}

template <bool PARTIALS, bool ROWA, int TM>
void launch_mode_tm(int mode, const Params& p, dim3 grid, hipStream_t stream) {
  const dim3 block(2 * TM);
  switch (mode) {
    case G64: hipLaunchKernelGGL((k_w4a4_gemm<PARTIALS, G64, ROWA, TM>), grid, block, 0, stream, p); return;
    case G128: hipLaunchKernelGGL((k_w4a4_gemm<PARTIALS, G128, ROWA, TM>), grid, block, 0, stream, p); return;
    default: hipLaunchKernelGGL((k_w4a4_gemm<PARTIALS, GBIG, ROWA, TM>), grid, block, 0, stream, p); return;
  }
}

// Tile height of the tiled kernel for M rows and smallest group gmin: 128 up
// to 128 rows (a 256-row tile would be half empty) and for g = 64 (its
// one-stage-ahead loads and per-k-step epilogue measured 6-10 % slower on 256
// rows at LLaMA-2-70B FFN shapes), else 256.
int tile_rows(int64_t M, int64_t gmin) { return M > 128 && gmin != 64 ? 256 : 128; }

// Waves per workgroup of the few-token kernels for an N-column output (the
// grid is one 32-column tile per workgroup): 8 below 512 workgroups, else 4.
int small_waves(int64_t tiles) { return tiles < 512 ? 8 : 4; }

// Few-token tile widths. The two widths split K between the waves alike (the
// wave count of the 32-column grid) and sum in the same order, so Y does not
// depend on the choice. 16 columns (k_w4a4_linear_small16) for the fused path
// wherever they apply: M <= 16, groups of 128 or more, per-group activation
// scales.
bool use_small16_fused(int64_t M, int64_t K, int64_t ga, int64_t gw) {
  const int64_t gmin = ga < gw ? ga : gw;
  return M <= SM16_TILE && gmin >= 128 && ga != K;
}
// The GEMM (k_w4a4_gemm_small16) likewise, except at M = 1 on a 32-column grid
// that spreads evenly over the 256 CUs (LLaMA-2-70B w2: 256 workgroups of 8
// waves, one per CU), which streams W faster there (measured 30.1 against
// 32.5 us; at M = 4 and 16 the 16-column tiles: 31.1 / 40.6 against 34.0 /
// 45.1 us).
bool use_small16(int64_t M, int64_t N, int64_t K, int64_t ga, int64_t gw) {
  const int64_t nwg = ((M + SM_TILE - 1) / SM_TILE) * ((N + SM_TILE - 1) / SM_TILE);
  return use_small16_fused(M, K, ga, gw) && (M > 1 || nwg % 256 != 0);
}

template <bool PARTIALS, bool ROWA>
void launch_mode(int mode, int tm, const Params& p, dim3 grid, hipStream_t stream) {
  if (tm == 256)
    launch_mode_tm<PARTIALS, ROWA, 256>(mode, p, grid, stream);
  else
    launch_mode_tm<PARTIALS, ROWA, 128>(mode, p, grid, stream);
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
  p.stages_per_split = (int)(g.K / BK);
  p.split_stride = 0;
  // Few tokens: the small-M path (32 x 32 tiles, K split between the waves of
  // a workgroup) when M <= 32, or M <= 64 and the grid (one tile row, N / 128
  // tiles) would hold fewer than 128 tiles (measured crossovers on the LLaMA-2-70B FFN shapes).
  const int64_t big_tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128);
  if (g.M <= 32 || (g.M <= 64 && big_tiles < 128)) {
    // waves per workgroup from the whole product's 32-column grid, so a
    // partials window runs the configuration the plain launch of this shape
    // runs, and both tile widths split K between the waves alike
    const int64_t nwg = ((g.M + SM_TILE - 1) / SM_TILE) * ((g.N + SM_TILE - 1) / SM_TILE);
    // 16-column tiles (see use_small16)
    if (use_small16(g.M, g.N, g.K, g.ga, g.gw)) {
      p.tile_m0 = (int)(g.m0 / SM16_TILE);
      p.tile_n0 = (int)(g.n0 / SM16_TILE);
      p.tiles_m = (int)((g.m0 + g.mc - 1) / SM16_TILE) - p.tile_m0 + 1;
      p.tiles_n = (int)((g.n0 + g.nc - 1) / SM16_TILE) - p.tile_n0 + 1;
      const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
      const int spg = (int)(gmin / 128);
      if (small_waves(nwg) == 8)
        launch_small16<8>(g, p, grid, spg, stream);
      else
        launch_small16<4>(g, p, grid, spg, stream);
      return;
    }
    p.tile_m0 = (int)(g.m0 / SM_TILE);
    p.tile_n0 = (int)(g.n0 / SM_TILE);
    p.tiles_m = (int)((g.m0 + g.mc - 1) / SM_TILE) - p.tile_m0 + 1;
    p.tiles_n = (int)((g.n0 + g.nc - 1) / SM_TILE) - p.tile_n0 + 1;
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    const int spg = (int)(gmin / 64);
    if (small_waves(nwg) == 8)
      launch_small<8>(g, p, grid, spg, stream);
    else
      launch_small<4>(g, p, grid, spg, stream);
    return;
  }
  // tile height from the whole product (a partials window gets the tiles the
  // plain launch of this shape runs)
  const int BM = tile_rows(g.M, gmin);
  p.tile_m0 = (int)(g.m0 / BM);
  p.tile_n0 = (int)(g.n0 / BN);
  p.tiles_m = (int)((g.m0 + g.mc - 1) / BM) - p.tile_m0 + 1;
  p.tiles_n = (int)((g.n0 + g.nc - 1) / BN) - p.tile_n0 + 1;
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  if (g.partials)
    launch_mode<true, false>(mode, BM, p, grid, stream);
  else if (g.ga == g.K)
    launch_mode<false, true>(mode, BM, p, grid, stream);
  else
    launch_mode<false, false>(mode, BM, p, grid, stream);
}

// LDS of a fused launch: the FP6 operand copy (24 bytes per 32 elements), the
// scales, and the cross-wave sum of the accumulators (16 floats per lane on
// 32-column tiles, 4 on 16-column tiles) for every wave but the first.
int64_t linear_small_lds_bytes(int64_t M, int64_t N, int64_t K, int64_t ga, int64_t gw) {
  const int nw = small_waves((N + SM_TILE - 1) / SM_TILE);
  const int acc = use_small16_fused(M, K, ga, gw) ? 4 : 16;
  return 24 * M * (K / 32) + 4 * M * (K / ga) + 4 * acc * 64 * (nw - 1);
}

template <int NW>
void launch_linear16_waves(int ga, dim3 grid, size_t lds, const LinParams& p, int spg, hipStream_t stream) {
  const dim3 block(64 * NW);
  switch (ga) {
    case 128: hipLaunchKernelGGL((k_w4a4_linear_small16<128, NW>), grid, block, lds, stream, p, spg); break;
    case 256: hipLaunchKernelGGL((k_w4a4_linear_small16<256, NW>), grid, block, lds, stream, p, spg); break;
    default: hipLaunchKernelGGL((k_w4a4_linear_small16<512, NW>), grid, block, lds, stream, p, spg); break;
  }
}

template <int NW>
void launch_linear_waves(int ga, dim3 grid, size_t lds, const LinParams& p, int spg, hipStream_t stream) {
  const dim3 block(64 * NW);
  switch (ga) {
    case 64: hipLaunchKernelGGL((k_w4a4_linear_small<64, NW>), grid, block, lds, stream, p, spg); break;
    case 128: hipLaunchKernelGGL((k_w4a4_linear_small<128, NW>), grid, block, lds, stream, p, spg); break;
    case 256: hipLaunchKernelGGL((k_w4a4_linear_small<256, NW>), grid, block, lds, stream, p, spg); break;
    default: hipLaunchKernelGGL((k_w4a4_linear_small<512, NW>), grid, block, lds, stream, p, spg); break;
  }
}

bool linear_small_supported(int64_t M, int64_t N, int64_t K, int64_t ga, int64_t gw) {
  if (M < 1 || M > SM_TILE || N < 1) return false;
  if (ga != 64 && ga != 128 && ga != 256 && ga != 512) return false;
  if (K % ga || K % gw || K % 128) return false;
  const int64_t gmin = ga < gw ? ga : gw;
  if ((ga > gw ? ga : gw) % gmin) return false;
  return linear_small_lds_bytes(M, N, K, ga, gw) <= kLinearSmallLds;
}

void launch_w4a4_linear_small(const void* x, int64_t M, int64_t K, int64_t ldx, int ga, const uint8_t* wq,
                              const float* ws, int gw, int64_t N, void* y, int ydtype, int64_t ldy,
                              hipStream_t stream) {
  LinParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.ldx = ldx;
  p.w = wq;
  p.sw = ws;
  p.sha = scale_shift(ga, K);
  p.shw = scale_shift(gw, K);
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.y = y;
  p.ydtype = ydtype;
  p.ldy = ldy;
  const int64_t gmin = ga < gw ? ga : gw;
  const int spg = (int)(gmin / 64);
  const int tiles_n = (int)((N + SM_TILE - 1) / SM_TILE);
  const size_t lds = (size_t)linear_small_lds_bytes(M, N, K, ga, gw);
  // the wave count of the few-token GEMM of this shape (from its 32-column
  // grid), so the waves' K ranges and the fixed-order sum of their
  // accumulators are the same whichever tile width either path takes
  if (use_small16_fused(M, K, ga, gw)) {
    const dim3 grid16((unsigned)((N + SM16_TILE - 1) / SM16_TILE));
    if (small_waves(tiles_n) == 8)
      launch_linear16_waves<8>(ga, grid16, lds, p, (int)(gmin / 128), stream);
    else
      launch_linear16_waves<4>(ga, grid16, lds, p, (int)(gmin / 128), stream);
    return;
  }
  const dim3 grid((unsigned)tiles_n);
  if (small_waves(tiles_n) == 8)
    launch_linear_waves<8>(ga, grid, lds, p, spg, stream);
  else
    launch_linear_waves<4>(ga, grid, lds, p, spg, stream);
}

SplitPlan plan_w4a4_splitk(int64_t M, int64_t N, int64_t K, int ga, int gw, int requested) {
  const int64_t nk = K / BK;
  const int64_t gmin = ga < gw ? ga : gw;
  const int64_t unit = gmin > BK ? gmin / BK : 1;        // stages per group: splits fall on group edges
  const int64_t units = nk / unit;
  const int BM = tile_rows(M, gmin);
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int64_t want = requested;
  if (want <= 0) {
    // enough workgroups for every slot of the chip (one 256-row or two
    // 128-row tiles per CU) when the tile grid alone leaves them idle; the
    // few-token path needs no split
    const int64_t slots = BM == 256 ? 256 : 512;
    const bool small_path = M <= 32 || (M <= 64 && tiles < 128);
    want = (small_path || tiles * 2 > slots) ? 1 : slots / tiles;
  }
  want = want < 1 ? 1 : want > units ? units : want;
  SplitPlan pl;
  pl.stages_per_split = (int)(((units + want - 1) / want) * unit);
  pl.splits = (int)((nk + pl.stages_per_split - 1) / pl.stages_per_split);
  return pl;
}

void launch_w4a4_gemm_splitk(const GemmArgs& g, const SplitPlan& pl, float* ws, hipStream_t stream) {
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
  p.y = ws;                      // split s writes fp32 ws[s][M][N]
  p.ydtype = 0;
  p.ldy = g.N;
  p.m0 = 0;
  p.mc = (int)g.M;
  p.n0 = 0;
  p.nc = (int)g.N;
  p.partials = nullptr;
  p.stages_per_split = pl.stages_per_split;
  p.split_stride = g.M * g.N;
  p.tile_m0 = 0;
  p.tile_n0 = 0;
  const int BM = tile_rows(g.M, gmin);
  p.tiles_m = (int)((g.M + BM - 1) / BM);
  p.tiles_n = (int)((g.N + BN - 1) / BN);
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n * pl.splits));
  if (g.ga == g.K)
    launch_mode<false, true>(mode, BM, p, grid, stream);
  else
    launch_mode<false, false>(mode, BM, p, grid, stream);
  const int64_t work = g.M * ((g.N & 3) == 0 ? g.N / 4 : g.N);
  const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 8192);
  hipLaunchKernelGGL(k_splitk_reduce, dim3(blocks), dim3(256), 0, stream, ws, pl.splits, (int)g.M, (int)g.N,
                     p.split_stride, g.y, g.ydtype, g.ldy);
}

}  // namespace w4a4
