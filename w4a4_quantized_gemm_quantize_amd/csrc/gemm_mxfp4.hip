// MXFP4 GEMM for gfx950 on the block-scaled FP4 matrix-core path.
//
// MXFP4 = FP4 E2M1 elements with one E8M0 scale per 32 along K (the
// "open-standard MXFP4" of the FP4 RL abstract; block rule of OCP MX v1.0).
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operand formats set to FP4
// multiplies a 32 x 64 A tile by a 64 x 32 B tile; lane l supplies the 32
// consecutive K codes (16 bytes) of row l%32, 32-block l/32, and the E8M0 byte
// of exactly that block, so the block scales are applied inside the
// instruction and accumulation is fp32 with no vector-unit epilogue. The kernel
// is tiled for the matrix cores: each wave owns a (BM/WM) x (BN/WN) output
// tile. When K % 256 == 0 the launch uses 256 x 256 workgroup tiles of 2 x 4
// waves (128 x 64 each: 8 MFMAs per 6 operand reads per 64-k step), 256-deep K
// stages and one workgroup per CU (2 waves per SIMD); otherwise 128 x 128
// tiles of 2 x 2 waves with 128-deep stages. On gfx950 the cost per flop that
// mattered most, in the order found: accumulator copies at stage boundaries
// (gone with the loop unrolled by the ring depth), L2 requests for row-major
// scales (gone with the panel layout), L2 and LDS bytes per flop (cut by the
// larger tile) and LDS bank conflicts (gone with the 64-bank swizzle below).
//
// Stages are fed through an LDS ring by direct global->LDS loads (no staging
// registers): 2 x 68 KB stages for the 256 x 256 tile (one stage in flight
// behind the matrix work), 3 x 34 KB for the 128 x 128 tile (two in flight).
// The debug-partials variant runs the same instruction one 32-block at a time
// with unit scales. Grids with more 256 x 256 tiles than CUs run a persistent
// variant: one workgroup per CU takes tile after tile and the ring runs on
// across tile edges, so a tile's Y stores drain under the next tile's first
// stages instead of every workgroup of a round writing its Y at once and
// refilling its ring from nothing.
//
// 32x32 MFMA output layout: D element r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
// col l%32.
#include <utility>

#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFmtFp4 = 4;       // cbsz / blgp operand format code for FP4 E2M1
constexpr int kUnitScale = 127;  // E8M0 byte of 2^0
constexpr int kGroupRows = 4;    // tile-rows per raster group

struct Params {
  const uint8_t* a;
  const uint8_t* ea;
  const uint8_t* w;
  const uint8_t* ew;
  int M, N, K;
  void* y;
  int ydtype;
  int64_t ldy;
  int tiles_m, tiles_n;
  int tile_m0, tile_n0;
  int m0, mc, n0, nc;
  int32_t* partials;
};

__device__ __forceinline__ v8i as_operand(uint4 v) {
  return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

typedef __attribute__((address_space(3))) void* lds_vptr;

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>) in order: a
// loop unrolled by construction (the step index stays a constant expression,
// e.g. for the instruction's immediate byte select), whatever the body's size.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Direct buffer -> LDS copies: lane l's 16 (4) bytes from base + voff + soff
// land at lds + 16 l (4 l). The buffer (MUBUF) form, unlike the global (FLAT)
// form, lets the compiler keep exact LDS-read wait counts while these loads
// are in flight, so operand reads of the next k-step overlap the MFMAs.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt on vmcnt only (expcnt/lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup tile BM x BN; waves in a WM x WN grid, each (BM/WM) x (BN/WN) =
// TI x TJ blocks of 32 x 32; K stage KB (128 or 256). S-stage LDS ring filled by
// direct global->LDS loads: stage kt+S-1 is in flight while stage kt is
// computed. A stage holds BM + BN rows of RB = KB/2 packed bytes (row-major, no
// pad: each wave-wide 1 KB load covers 1024/RB rows) and KB/128 E8M0 dwords per
// row. A 256-deep stage makes each row's piece a whole 128-byte line, so the L2
// serves line-sized requests instead of 64-byte halves. The LDS serves a
// 16-byte read for 16 lanes per clock (64 banks of 4 bytes): the SL = RB/16
// slots of a row are XOR-swizzled with (row >> log2(16/SL)) & (SL-1) so the 16
// lanes that read one slot of 16 consecutive rows hit 16 distinct 16-byte bank
// groups.
template <int BM, int BN, int WM, int WN, int KB, int S, bool PARTIALS, bool PERSIST, int YT>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_mxfp4_gemm(Params p) {
  static_assert(S == 2 || S == 3, "ring depth");    // stages in LDS; S - 1 in flight
  constexpr int D = S - 1;                          // prefetch distance in stages
  constexpr int NWAVE = WM * WN;
  constexpr int RB = KB / 2;                        // packed bytes per row per stage
  constexpr int SL = RB / 16;                       // 16-byte slots per row
  constexpr int RPK = 1024 / RB;                    // rows per 1 KB load
  constexpr int SWS = SL == 4 ? 2 : 1;              // log2(16 / SL)
  constexpr int NSTEP = KB / 64;                    // MFMA k-steps per stage
  constexpr int NEW = 2;                            // E8M0 dwords per row per stage (a panel row)
  constexpr int TI = BM / WM / 32, TJ = BN / WN / 32;   // 32x32 blocks per wave
  constexpr int NA = BM / RPK / NWAVE, NW = BN / RPK / NWAVE;   // 1 KB loads per wave per stage
  constexpr int NE = (NEW * (BM + BN) + 64 * NWAVE - 1) / (64 * NWAVE); // scale-dword loads per wave
  constexpr int W_OFF = BM * RB;
  constexpr int E_OFF = (BM + BN) * RB;
  constexpr int STAGE = E_OFF + NE * NWAVE * 64 * 4;
  constexpr int PER_STAGE = NA + NW + NE;           // load instructions per wave per stage
  static_assert(KB == 128 || KB == 256, "stage depth");
  static_assert(NA * RPK * NWAVE == BM && NW * RPK * NWAVE == BN, "tile rows per wave");
  // One array per ring slot (the loop is unrolled by S, so every access names
  // its slot): the compiler can then tell an in-flight load into one slot from
  // LDS reads of another and does not wait for it.
  __shared__ __align__(16) uint8_t sm0[STAGE];
  __shared__ __align__(16) uint8_t sm1[STAGE];
  __shared__ __align__(16) uint8_t sm2[S == 3 ? STAGE : 16];

  const int nblk = p.tiles_m * p.tiles_n;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int row_bytes = p.K >> 1;
  const int nk = p.K / KB;
  const int lrow = lane / SL, lslot = lane % SL;

  // ---- the tile of logical index t: its origin, buffer resources over its
  // rows (row offsets stay 32-bit; the host limits K so a tile's rows span
  // < 2^31 bytes) and per-lane row offsets. Consecutive indices on one XCD
  // (t % 8) take consecutive tiles of a raster of kGroupRows tile-rows.
  int tile_m, tile_n, a_rows, w_rows;
  __amdgpu_buffer_rsrc_t rA, rW;
  int voffA[NA], voffW[NW];
  constexpr int CA = NEW * BM / 64, CW = NEW * BN / 64;   // scale chunks per stage
  static_assert(CA * 64 == NEW * BM && CW * 64 == NEW * BN, "scale chunks");
  int voffE[NE], voffE4[NE];    // the lane's offset in an 8-byte / 4-byte pitch scale panel
  auto setup = [&](int t) {
    int bid = t;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int per_group = kGroupRows * p.tiles_n;
    const int grp = bid / per_group;
    const int first_m = grp * kGroupRows;
    const int gsize = min(p.tiles_m - first_m, kGroupRows);
    const int rem = bid - grp * per_group;
    tile_m = (p.tile_m0 + first_m + rem % gsize) * BM;
    tile_n = (p.tile_n0 + rem / gsize) * BN;
    a_rows = min(BM, p.M - tile_m);
    w_rows = min(BN, p.N - tile_n);
    rA = buffer_rsrc(p.a + (int64_t)tile_m * row_bytes, a_rows * row_bytes);
    rW = buffer_rsrc(p.w + (int64_t)tile_n * row_bytes, w_rows * row_bytes);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = RPK * (wave + NWAVE * i) + lrow;
      const int seg = lslot ^ ((row >> SWS) & (SL - 1));
      voffA[i] = min(row, a_rows - 1) * row_bytes + 16 * seg;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int row = RPK * (wave + NWAVE * i) + lrow;
      const int seg = lslot ^ ((row >> SWS) & (SL - 1));
      voffW[i] = min(row, w_rows - 1) * row_bytes + 16 * seg;
    }
    // Scale dword e = NEW * r + w of a stage is dword w of the stage's scales
    // of A row r (e < NEW * BM) or of W row r - BM; each wave load moves one
    // 64-dword chunk of them, chunk c = NE * wave + j.
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int c = NE * wave + j;
      const bool is_a = c < CA;
      const int e = 64 * (is_a ? c : c - CA) + lane;
      const int r = min(e / NEW, (is_a ? a_rows : w_rows) - 1), w = e % NEW;
      voffE[j] = 8 * r + 4 * w;
      voffE4[j] = 4 * r;
    }
  };
  // Scales are stored in panels of 8 blocks (256 k): panel q holds, row after
  // row, each row's 8 scale bytes of blocks 8q..8q+7 (a last panel of 4 blocks
  // holds 4 bytes per row); consecutive lanes read consecutive dwords of one
  // panel. A buffer resource is uniform, so a chunk lies wholly in the A part
  // or the W part.
  // a K that is 128 mod 256 ends in a 4-block panel (4 scale bytes per row)
  const bool half_tail = (p.K & 255) != 0;
  // Scale chunk j of stage kt: the rows of panel kt (KB = 256) or of panel
  // kt / 2 (KB = 128, both halves of a panel read its whole rows); a last
  // 4-block panel has 4-byte rows, read into both dwords of a row slot. Chunks
  // beyond the stage's (none in the shipped tile shapes) re-read chunk 0's
  // dwords into their own unused LDS words, so every wave issues the same
  // number of loads per stage (the vmcnt waits count on it).
  auto issue_scales = [&](int j, int kt, uint8_t* lds) {
    const int c = NE * wave + j;
    const bool is_a = c < CA || c >= CA + CW;
    const uint8_t* mat = is_a ? p.ea : p.ew;
    const int64_t rows_all = is_a ? p.M : p.N;
    const int t0 = is_a ? tile_m : tile_n;
    const int nrow = is_a ? a_rows : w_rows;
    if constexpr (KB == 256) {
      dma4(buffer_rsrc(mat + 8 * rows_all * kt + 8 * t0, 8 * nrow), voffE[j], 0, lds);
    } else {
      const uint8_t* panel = mat + 8 * rows_all * (kt >> 1);
      if (half_tail && kt == nk - 1)
        dma4(buffer_rsrc(panel + 4 * t0, 4 * nrow), voffE4[j], 0, lds);
      else
        dma4(buffer_rsrc(panel + 8 * t0, 8 * nrow), voffE[j], 0, lds);
    }
  };
#define ISSUE(KT, SM)                                                                \
  {                                                                                  \
    uint8_t* base_ = (SM);                                                           \
    _Pragma("unroll") for (int i = 0; i < NA; ++i)                                   \
        dma16(rA, voffA[i], (KT) * RB, base_ + (wave + NWAVE * i) * 1024);         \
    _Pragma("unroll") for (int i = 0; i < NW; ++i)                                   \
        dma16(rW, voffW[i], (KT) * RB, base_ + W_OFF + (wave + NWAVE * i) * 1024); \
    _Pragma("unroll") for (int j = 0; j < NE; ++j)                                   \
        issue_scales(j, (KT), base_ + E_OFF + (NE * wave + j) * 256);              \
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
  int offA[NSTEP], offW[NSTEP];
#pragma unroll
  for (int u = 0; u < NSTEP; ++u) {
    offA[u] = rowA * RB + 16 * ((2 * u + lhi) ^ ((rowA >> SWS) & (SL - 1)));
    offW[u] = rowW * RB + 16 * ((2 * u + lhi) ^ ((rowW >> SWS) & (SL - 1)));
  }
  // Operands of two 64-k steps (FP4: 16 bytes per lane): step u + 1 is read
  // from LDS while the MFMAs of step u run.
  uint4 av[2][TI], wv[2][TJ];
  // The lane's scale dword per operand row block, once per stage: within a
  // panel row the even blocks' bytes come first, then the odd ones', so dword
  // l/32 of the row holds the bytes of all 32-blocks this lane feeds and step
  // U selects byte U with the instruction's byte select (shifted by 16 bits
  // for the second half of a panel in 128-deep stages, and in a 4-byte last
  // panel row for the odd lanes).
  int ea[TI], ew[TJ];

// Operands of one 64-k MFMA step U from ring slot SM: lane l feeds 32-block
// 2U + l/32 of the stage in its row. The swizzle term of row + 32 i equals
// that of row, so one base per step serves every row block i.
#define LOAD_OPS(SM, U, B)                                                            \
  {                                                                                  \
    const uint8_t* st_ = (SM);                                                       \
    _Pragma("unroll") for (int i = 0; i < TI; ++i) {                                 \
      av[B][i] = *reinterpret_cast<const uint4*>(st_ + offA[U] + 32 * RB * i);      \
    }                                                                                \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j) {                                 \
      wv[B][j] = *reinterpret_cast<const uint4*>(st_ + W_OFF + offW[U] + 32 * RB * j); \
    }                                                                                \
  }
// Matrix work of step U of stage KT. The partials variant runs one 32-block at
// a time with unit scales, so D = sum va*vw over that block exactly.
#define MMA_STEP(KT, U, B)                                                           \
  {                                                                                  \
    if constexpr (PARTIALS) {                                                        \
      const v8i zero_ = v8i{0, 0, 0, 0, 0, 0, 0, 0};                                 \
      _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                \
        const int gblk = (KB / 32) * (KT) + 2 * (U) + h;                             \
        _Pragma("unroll") for (int i = 0; i < TI; ++i)                               \
        _Pragma("unroll") for (int j = 0; j < TJ; ++j) {                             \
          v16f zacc;                                                                 \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) zacc[r] = 0.0f;             \
          const v16f d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(            \
              lhi == h ? as_operand(av[B][i]) : zero_, lhi == h ? as_operand(wv[B][j]) : zero_, zacc, \
              kFmtFp4, kFmtFp4, 0, kUnitScale, 0, kUnitScale);                       \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) {                           \
            const int m = tile_m + wm * (BM / WM) + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3); \
            const int n = tile_n + wn * (BN / WN) + 32 * j + l32;                     \
            if (m >= p.m0 && m < p.m0 + p.mc && n >= p.n0 && n < p.n0 + p.nc)        \
              p.partials[((int64_t)gblk * p.mc + (m - p.m0)) * p.nc + (n - p.n0)] = (int32_t)(d[r] * 4.0f); \
          }                                                                          \
        }                                                                            \
      }                                                                              \
    } else {                                                                         \
      MMA_SEL(B, U) /* U is a constant: the byte select is an immediate */           \
    }                                                                                \
  }
#define MMA_SEL(B, SEL)                                                              \
  _Pragma("unroll") for (int i = 0; i < TI; ++i)                                     \
  _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                     \
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                     \
        as_operand(av[B][i]), as_operand(wv[B][j]), acc[i][j], kFmtFp4, kFmtFp4, SEL, ea[i], SEL, ew[j]);
// The stage's scale dwords (see ea / ew).
#define LOAD_SCALES(KT, SM)                                                          \
  {                                                                                  \
    const uint32_t* se_ = reinterpret_cast<const uint32_t*>((SM) + E_OFF);           \
    const bool tail_ = KB == 128 && half_tail && (KT) == nk - 1;                     \
    const int sh_ = KB == 256 ? 0 : tail_ ? 16 * lhi : 16 * ((KT) & 1);             \
    const int w_ = tail_ ? 0 : lhi;                                                  \
    _Pragma("unroll") for (int i = 0; i < TI; ++i)                                   \
      ea[i] = (int)(se_[NEW * (rowA + 32 * i) + w_] >> sh_);                         \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                   \
      ew[j] = (int)(se_[NEW * (BM + rowW + 32 * j) + w_] >> sh_);                    \
  }
// Keeps the next step's LDS reads ahead of this step's MFMAs.
#ifndef PIPE_FENCE_ON
#define PIPE_FENCE_ON 1
#endif
#define PIPE_FENCE()                                                    \
  {                                                                     \
    if (PIPE_FENCE_ON) __builtin_amdgcn_sched_barrier(0);               \
  }
// Barrier between ring stages. Each wave has already waited for its own
// direct loads of the stage (vmcnt), so after the barrier every wave's part of
// the stage is in LDS, and every wave has finished reading the slot about to be
// refilled. No memory fence: a fence would also drain the loads still in
// flight for later stages. The scheduling barrier keeps the compiler from
// moving LDS accesses across it.
#define STAGE_BARRIER()                                                 \
  {                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                  \
    __builtin_amdgcn_s_barrier();                                       \
    __builtin_amdgcn_sched_barrier(0);                                  \
  }
// Iteration for stage KT held in slot CUR; stage KT+D is issued into slot NXT
// (the slot stage KT-1 used, free once every wave has passed the barrier) after
// the first step's operand reads, so those reads never wait behind the new loads.
// At the top, stages KT .. KT+D-1 are in flight; the wait leaves the later
// D-1 of them outstanding.
#define ITER(KT, CUR, NXT)                                              \
  {                                                                     \
    if (D == 2 && (KT) + 1 < nk) wait_vmcnt<(D - 1) * PER_STAGE>();     \
    else wait_vmcnt<0>();                                               \
    STAGE_BARRIER();                                                    \
    LOAD_SCALES(KT, CUR);                                               \
    LOAD_OPS(CUR, 0, 0);                                                \
    if ((KT) + D < nk) ISSUE((KT) + D, NXT);                            \
    static_for<NSTEP>([&](auto uc_) {                                   \
      constexpr int u_ = decltype(uc_)::value;                          \
      if constexpr (u_ + 1 < NSTEP) LOAD_OPS(CUR, u_ + 1, (u_ + 1) & 1); \
      PIPE_FENCE();                                                     \
      MMA_STEP(KT, u_, u_ & 1);                                         \
      PIPE_FENCE();                                                     \
    });                                                                 \
  }

  // Y stores of a finished tile with origin (tm, tn) and am valid rows. The
  // persistent kernel takes only the full-tile path (its host side admits
  // only M a multiple of BM): TI * TJ * 16 store instructions per wave.
  auto store_tile = [&](int tm, int tn, int am) {
    const int ydt = YT >= 0 ? YT : p.ydtype;      // Y dtype: fixed by YT >= 0, else from the call
    const int esz = ydt == 0 ? 4 : 2;
    if (!PERSIST && (am != BM || (int64_t)BM * p.ldy * esz >= (int64_t{1} << 31))) {
      // last row tile of a ragged M (or a huge ldy): per-element checked stores
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = tm + wm * (BM / WM) + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3);
            const int n = tn + wn * (BN / WN) + 32 * j + l32;
            if (m < p.M && n < p.N) {
              if (ydt == 0)
                static_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = acc[i][j][r];
              else
                static_cast<__half*>(p.y)[(int64_t)m * p.ldy + n] = __float2half_rn(acc[i][j][r]);
            }
          }
      return;
    }
    // Every row of the tile is valid and the tile spans < 2^31 bytes: buffer
    // stores with each register's row offset in the scalar offset. A lane
    // whose column is >= N gets a vector offset past the resource, so the
    // hardware drops its stores.
    const int ldb = (int)(p.ldy * esz);
    const __amdgpu_buffer_rsrc_t rY = buffer_rsrc(static_cast<uint8_t*>(p.y) + (int64_t)tm * ldb, BM * ldb);
    const int row0 = wm * (BM / WM) + 4 * lhi;       // tile row of register 0, block 0
    int voffY[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = tn + wn * (BN / WN) + 32 * j + l32;
      voffY[j] = n < p.N ? row0 * ldb + n * esz : kDroppedOffset;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int soff = (32 * i + 8 * (r >> 2) + (r & 3)) * ldb;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if (ydt == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rY, voffY[j], soff, kStoreNT);
          else
            __builtin_amdgcn_raw_buffer_store_b16(__half_as_ushort(__float2half_rn(acc[i][j][r])), rY, voffY[j],
                                                  soff, kStoreNT);
        }
      }
  };

  if constexpr (PERSIST) {
    // Persistent schedule: workgroup b takes tiles b, b + G, b + 2G, ... (G
    // workgroups, a multiple of 8, so all of them run on XCD b % 8) and the
    // ring runs on across tile edges (K in an even number >= 4 of stages, so
    // every tile starts in slot 0). During a tile's last stage the first
    // stage of its next tile is issued; after the last stage's matrix work
    // the second one; then the tile's Y stores. A wave's memory operations
    // complete in issue order and it keeps at most 63 in flight, so it issues
    // its last stores once the next tile's two stages and about half of the
    // stores are done; the other half drain under those two stages' matrix
    // work, and stage 2 waits for them. (Without this, every workgroup of a
    // round writes its Y at the same moment and then refills its ring from
    // nothing.) The first tile's first two stages are peeled and the tile
    // loop starts at the last stage, so at every join of the control flow the
    // same memory operations are in flight and the compiler's own waits for
    // the ring's loads count exactly as the ones written here.
    static_assert(S == 2 && !PARTIALS, "persistent schedule: 2-stage ring, Y output");
    // Y stores per wave per tile. The waits count at most 63 operations (the
    // counter's range; a wave does not issue beyond it): with in-order
    // completion a clamped wait waits for more, never for less. With 128
    // stores they clamp to no wait at all: once the stores are issued, at
    // most 63 operations are outstanding and the two stages issued before
    // them are complete.
    constexpr int NST = TI * TJ * 16;
    constexpr int W0 = PER_STAGE + NST < 63 ? PER_STAGE + NST : 63;
    constexpr int W1 = NST < 63 ? NST : 63;
    static_assert(PER_STAGE < 63, "vmcnt range");
    const int G = gridDim.x;
    int t = blockIdx.x;
// Stage 0 of a tile (slot 0; stage 1 already in flight into slot 1): wait
// until only the WAIT_ operations issued after stage 0 are outstanding.
#define STAGE0(WAIT_)                                                   \
  {                                                                     \
    wait_vmcnt<WAIT_>();                                                \
    STAGE_BARRIER();                                                    \
    LOAD_SCALES(0, sm0);                                                \
    LOAD_OPS(sm0, 0, 0);                                                \
    static_for<NSTEP>([&](auto uc_) {                                   \
      constexpr int u_ = decltype(uc_)::value;                          \
      if constexpr (u_ + 1 < NSTEP) LOAD_OPS(sm0, u_ + 1, (u_ + 1) & 1); \
      PIPE_FENCE();                                                     \
      MMA_STEP(0, u_, u_ & 1);                                          \
      PIPE_FENCE();                                                     \
    });                                                                 \
  }
// Stage 1 (slot 1; WAIT_ operations issued after it) issues stage 2, then
// the stages up to nk - 2 run as in the plain schedule.
#define STAGE1_TO_NK2(WAIT_)                                            \
  {                                                                     \
    wait_vmcnt<WAIT_>();                                                \
    STAGE_BARRIER();                                                    \
    LOAD_SCALES(1, sm1);                                                \
    LOAD_OPS(sm1, 0, 0);                                                \
    ISSUE(2, sm0);                                                      \
    static_for<NSTEP>([&](auto uc_) {                                   \
      constexpr int u_ = decltype(uc_)::value;                          \
      if constexpr (u_ + 1 < NSTEP) LOAD_OPS(sm1, u_ + 1, (u_ + 1) & 1); \
      PIPE_FENCE();                                                     \
      MMA_STEP(1, u_, u_ & 1);                                          \
      PIPE_FENCE();                                                     \
    });                                                                 \
    for (int kt = 2; kt < nk - 2; kt += 2) {                            \
      ITER(kt, sm0, sm1)                                                \
      ITER(kt + 1, sm1, sm0)                                            \
    }                                                                   \
    ITER(nk - 2, sm0, sm1)                                              \
  }
// The last stage (slot 1) of a tile; with NEXT, the first two stages of the
// next tile are issued (its setup done) around the matrix work.
#define LAST_STAGE(NEXT)                                                \
  {                                                                     \
    wait_vmcnt<0>();                                                    \
    STAGE_BARRIER();                                                    \
    LOAD_SCALES(nk - 1, sm1);                                           \
    LOAD_OPS(sm1, 0, 0);                                                \
    em = tile_m;                                                        \
    en = tile_n;                                                        \
    if constexpr (NEXT) {                                               \
      t += G;                                                           \
      setup(t);                                                         \
      ISSUE(0, sm0);                                                    \
    }                                                                   \
    static_for<NSTEP>([&](auto uc_) {                                   \
      constexpr int u_ = decltype(uc_)::value;                          \
      if constexpr (u_ + 1 < NSTEP) LOAD_OPS(sm1, u_ + 1, (u_ + 1) & 1); \
      PIPE_FENCE();                                                     \
      MMA_STEP(nk - 1, u_, u_ & 1);                                     \
      PIPE_FENCE();                                                     \
    });                                                                 \
    if constexpr (NEXT) {                                               \
      STAGE_BARRIER();                                                  \
      ISSUE(1, sm1);                                                    \
    }                                                                   \
    store_tile(em, en, BM);                                             \
  }
    // this workgroup's tile count: the tile loop runs a fixed number of
    // times, so no load is issued under a condition the compiler cannot
    // follow into the waits that depend on it
    const int ntile = (nblk - t + G - 1) / G;
    int em = 0, en = 0;
    setup(t);
    ISSUE(0, sm0);
    ISSUE(1, sm1);
    STAGE0(PER_STAGE)
    STAGE1_TO_NK2(0)
    for (int it = 1; it < ntile; ++it) {
      LAST_STAGE(true)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
      STAGE0(W0)
      STAGE1_TO_NK2(W1)
    }
    LAST_STAGE(false)
#undef LAST_STAGE
#undef STAGE0
#undef STAGE1_TO_NK2
  } else {
    setup(blockIdx.x);
    ISSUE(0, sm0);
    if (S == 3 && nk > 1) ISSUE(1, sm1);
    // Unrolled by the ring depth, so every stage names its slot statically and
    // the loop has one back edge: the accumulators stay in the registers the
    // matrix instructions write, with no copies between stages.
    if constexpr (S == 3) {
      for (int kt = 0;; kt += 3) {
        ITER(kt, sm0, sm2)
        if (kt + 1 >= nk) break;
        ITER(kt + 1, sm1, sm0)
        if (kt + 2 >= nk) break;
        ITER(kt + 2, sm2, sm1)
        if (kt + 3 >= nk) break;
      }
    } else {
      for (int kt = 0;; kt += 2) {
        ITER(kt, sm0, sm1)
        if (kt + 1 >= nk) break;
        ITER(kt + 1, sm1, sm0)
        if (kt + 2 >= nk) break;
      }
    }
    if constexpr (!PARTIALS) store_tile(tile_m, tile_n, a_rows);
  }
#undef ITER
#undef STAGE_BARRIER
#undef MMA_STEP
#undef LOAD_OPS
#undef LOAD_SCALES
#undef MMA_SEL
#undef ISSUE
}

// YT: the Y dtype fixed at compile time (0 fp32, 1 fp16), or -1 to read it
// from the call. The persistent kernel fixes it: its stores are then one
// straight-line block, which the compiler's wait counting follows exactly.
template <int BM, int BN, int WM, int WN, int KB, int S, bool PARTIALS, bool PERSIST, int YT>
void launch_cfg(Params p, const GemmArgs& g, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((k_mxfp4_gemm<BM, BN, WM, WN, KB, S, PARTIALS, PERSIST, YT>), dim3(grid), dim3(64 * WM * WN),
                     0, stream, p);
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// 256 x 256 tiles (2 x 4 waves of 128 x 64) with 256-deep stages in a 2-stage
// ring (2 x 68 KB) when K allows, else 128 x 128 tiles (2 x 2 waves) with
// 128-deep stages in a 3-stage ring. The 256 x 256 kernel runs the persistent
// schedule (one workgroup per CU, the ring running on across tiles) when the
// grid holds more tiles than CUs, every row tile is full (M a multiple of
// 256) and K is an even number >= 4 of 256-deep stages.
template <bool PARTIALS>
void launch_for(Params p, const GemmArgs& g, hipStream_t stream) {
  const int esz = g.ydtype == 0 ? 4 : 2;
  const int64_t ldb = g.ldy * esz;
  if (g.K % 256 == 0) {
    constexpr int BM = 256, BN = 256;
    p.tile_m0 = (int)(g.m0 / BM);
    p.tile_n0 = (int)(g.n0 / BN);
    p.tiles_m = (int)((g.m0 + g.mc - 1) / BM) - p.tile_m0 + 1;
    p.tiles_n = (int)((g.n0 + g.nc - 1) / BN) - p.tile_n0 + 1;
    const int64_t nblk = (int64_t)p.tiles_m * p.tiles_n;
    if constexpr (!PARTIALS) {
      const int64_t slots = cu_count() / 8 * 8;
      const int64_t nk = g.K / 256;
      if (slots >= 8 && nblk > slots && g.M % BM == 0 && nk >= 4 && nk % 2 == 0 &&
          BM * ldb < (int64_t{1} << 31)) {
        if (g.ydtype == 0)
          launch_cfg<256, 256, 2, 4, 256, 2, false, true, 0>(p, g, (unsigned)slots, stream);
        else
          launch_cfg<256, 256, 2, 4, 256, 2, false, true, 1>(p, g, (unsigned)slots, stream);
        return;
      }
    }
    launch_cfg<256, 256, 2, 4, 256, 2, PARTIALS, false, -1>(p, g, (unsigned)nblk, stream);
  } else {
    constexpr int BM = 128, BN = 128;
    p.tile_m0 = (int)(g.m0 / BM);
    p.tile_n0 = (int)(g.n0 / BN);
    p.tiles_m = (int)((g.m0 + g.mc - 1) / BM) - p.tile_m0 + 1;
    p.tiles_n = (int)((g.n0 + g.nc - 1) / BN) - p.tile_n0 + 1;
    launch_cfg<128, 128, 2, 2, 128, 3, PARTIALS, false, -1>(p, g, (unsigned)(p.tiles_m * p.tiles_n), stream);
  }
}

}  // namespace

void launch_mxfp4_gemm(const GemmArgs& g, hipStream_t stream) {
  Params p;
  p.a = g.a;
  p.ea = static_cast<const uint8_t*>(g.sa);
  p.w = g.w;
  p.ew = static_cast<const uint8_t*>(g.sw);
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
  if (g.partials)
    launch_for<true>(p, g, stream);
  else
    launch_for<false>(p, g, stream);
}

}  // namespace w4a4
