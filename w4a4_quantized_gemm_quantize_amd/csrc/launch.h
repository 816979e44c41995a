// Internal launchers behind the C ABI. Arguments are validated by the caller
// (api.hip); these only pick a kernel configuration and enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

void launch_int4_quant(const void* x, int64_t M, int64_t K, int64_t ldx, int group,
                       uint8_t* q, float* s, hipStream_t stream);

// mode 0: MXFP4 codes of x; 1: [Q(x) | Q(x - deq Q(x))] along K (width 2K);
// 2: [Q(x) | Q(x)] (width 2K); 3: as 1 with the second scale tied to the
// first (first exponent: nothing clips; second: the first minus 2)
void launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ldx,
                        uint8_t* q, uint8_t* e8m0, int mode, hipStream_t stream);

// Window [m0, m0+mc) x [n0, n0+nc); for the plain GEMM the window is the whole
// output and partials == nullptr.
struct GemmArgs {
  const uint8_t* a;
  const void* sa;      // float* (INT4) or uint8_t* (MXFP4, NVFP4)
  const uint8_t* w;
  const void* sw;
  int ga, gw;          // INT4 group sizes (unused for MXFP4)
  int64_t M, N, K;
  void* y;
  int ydtype;
  int64_t ldy;
  int64_t m0, mc, n0, nc;
  int32_t* partials;
};

void launch_w4a4_gemm(const GemmArgs& a, hipStream_t stream);

// K split of the tiled W4A4 GEMM: `splits` workgroups per output tile, each
// over `stages_per_split` 128-k stages (whole groups), fp32 partial outputs in
// a workspace [splits][M][N], summed in split order into y.
struct SplitPlan {
  int splits;
  int stages_per_split;
};
// requested <= 0: enough splits to fill the chip when the tile grid does not
SplitPlan plan_w4a4_splitk(int64_t M, int64_t N, int64_t K, int ga, int gw, int requested);
void launch_w4a4_gemm_splitk(const GemmArgs& a, const SplitPlan& plan, float* workspace, hipStream_t stream);
void launch_mxfp4_gemm(const GemmArgs& a, hipStream_t stream);

// Fused decode path: activation quantization in the few-token GEMM (one
// launch). Supported when M <= 32, the activation group is 64/128/256/512 and
// the workgroup's LDS copy of the quantized activations fits kLinearSmallLds.
constexpr int64_t kLinearSmallLds = 64 * 1024;
bool linear_small_supported(int64_t M, int64_t N, int64_t K, int64_t ga, int64_t gw);
void launch_w4a4_linear_small(const void* x, int64_t M, int64_t K, int64_t ldx, int ga, const uint8_t* wq,
                              const float* ws, int gw, int64_t N, void* y, int ydtype, int64_t ldy,
                              hipStream_t stream);

// NVFP4: *gscale = fl32(max|x| / 2688) (0 for rows == 0)
void launch_nvfp4_global_scale(const void* x, int64_t rows, int64_t K, int64_t ldx, float* gscale,
                               hipStream_t stream);
void launch_nvfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ldx, const float* gscale,
                        uint8_t* q, uint8_t* scales, hipStream_t stream);
// a.sa / a.sw: E4M3 panel scales; ga, gw: device pointers to the global scales
// (unused by the partials export)
void launch_nvfp4_gemm(const GemmArgs& a, const float* ga, const float* gw, hipStream_t stream);

// Storage conversions (layout.hip). count: device int32 receiving the number
// of -8 codes (none may be NULL: not counted).
void launch_repack_int4(const uint8_t* nibbles, int64_t rows, int64_t K, uint8_t* packed, int32_t* count,
                        hipStream_t stream);
void launch_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, uint8_t* nibbles, hipStream_t stream);
void launch_transpose_f32(const float* in, int64_t rows, int64_t cols, float* out, hipStream_t stream);
// fmt 0: E8M0 (blocks of 32), 1: E4M3 (blocks of 16); nb = blocks per row
void launch_scale_panels(int fmt, bool to_panels, const uint8_t* in, int64_t rows, int64_t nb, uint8_t* out,
                         hipStream_t stream);

}  // namespace w4a4
