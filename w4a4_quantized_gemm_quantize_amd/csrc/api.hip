// C ABI of libw4a4: argument validation, then one kernel launch per call.
// The contract of each entry point is documented in include/w4a4.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"
#include "w4a4.h"

using w4a4::GemmArgs;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

w4a4_status_t launched() {
  return hipGetLastError() == hipSuccess ? W4A4_OK : W4A4_E_HIP;
}

// Quantizer groups: 64/128/256/512 or the whole row.
bool quant_group_ok(int64_t K, int32_t group) {
  if (group == K) return true;
  if (group != 64 && group != 128 && group != 256 && group != 512) return false;
  return K % group == 0;
}

// GEMM groups: a power of two >= 64 dividing K, or K itself (per token); nested.
bool gemm_group_ok(int64_t K, int32_t g) {
  if (g == K) return true;
  return g >= 64 && (g & (g - 1)) == 0 && K % g == 0;
}

// The finer group bounds the fp32 partials: |P_b| <= 49 g must stay below 2^24
// for them to be exact integers.
constexpr int32_t kMaxPartialGroup = 1 << 18;

// Longest K of the INT4 GEMM: a 256-row tile of packed codes (K / 2 bytes per
// row) must span < 2^31 bytes for the kernel's 32-bit buffer offsets.
constexpr int64_t kMaxGemmK = int64_t{1} << 23;

bool gemm_groups_ok(int64_t K, int32_t ga, int32_t gw) {
  if (!gemm_group_ok(K, ga) || !gemm_group_ok(K, gw)) return false;
  const int32_t lo = ga < gw ? ga : gw, hi = ga < gw ? gw : ga;
  return hi % lo == 0 && lo <= kMaxPartialGroup;
}

w4a4_status_t check_y(void* y, int32_t ydt, int64_t N, int64_t ldy) {
  if (ydt != W4A4_Y_F32 && ydt != W4A4_Y_F16) return W4A4_E_DTYPE;
  if (ldy < N) return W4A4_E_SHAPE;
  if (!y) return W4A4_E_NULL;
  if (!aligned(y, ydt == W4A4_Y_F32 ? 4 : 2)) return W4A4_E_ALIGN;
  return W4A4_OK;
}

w4a4_status_t check_window(int64_t M, int64_t N, int64_t m0, int64_t mc, int64_t n0, int64_t nc) {
  if (mc <= 0 || nc <= 0 || m0 < 0 || n0 < 0 || m0 + mc > M || n0 + nc > N) return W4A4_E_SHAPE;
  return W4A4_OK;
}

}  // namespace

extern "C" {

const char* w4a4_status_str(int status) {
  switch (status) {
    case W4A4_OK: return "ok";
    case W4A4_E_NULL: return "null pointer";
    case W4A4_E_SHAPE: return "unsupported shape or leading dimension";
    case W4A4_E_GROUP: return "unsupported or non-nesting group size";
    case W4A4_E_ALIGN: return "misaligned pointer or leading dimension";
    case W4A4_E_DTYPE: return "unknown output dtype";
    case W4A4_E_HIP: return "HIP launch error";
    case W4A4_E_SCRATCH: return "needs more scratch memory than the library's static buffer holds";
    default: return "unknown status";
  }
}

w4a4_status_t w4a4_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, int32_t group,
                                uint8_t* xq, float* xs, void* stream) {
  if (M < 0 || K <= 0 || K % 16 || ldx < K) return W4A4_E_SHAPE;
  if (!quant_group_ok(K, group)) return W4A4_E_GROUP;
  if (ldx % 8) return W4A4_E_ALIGN;
  if (M == 0) return W4A4_OK;
  if (!x || !xq || !xs) return W4A4_E_NULL;
  if (!aligned(x, 16) || !aligned(xq, 8) || !aligned(xs, 4)) return W4A4_E_ALIGN;
  w4a4::launch_int4_quant(x, M, K, ldx, group, xq, xs, as_stream(stream));
  return launched();
}

w4a4_status_t w4a4_pack_weight(const void* w, int64_t N, int64_t K, int32_t group,
                               uint8_t* wq, float* ws, void* stream) {
  return w4a4_quantize_act(w, N, K, K, group, wq, ws, stream);
}

static w4a4_status_t gemm_common(const uint8_t* xq, const float* xs, int32_t ga,
                                 const uint8_t* wq, const float* ws, int32_t gw,
                                 int64_t M, int64_t N, int64_t K, GemmArgs& g) {
  // K <= 2^23: a 256-row tile then spans <= 2^30 bytes, within the kernel's
  // signed 32-bit buffer sizes and offsets
  if (M < 0 || N < 0 || K <= 0 || K % 128 || K > kMaxGemmK) return W4A4_E_SHAPE;
  if (!gemm_groups_ok(K, ga, gw)) return W4A4_E_GROUP;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!xq || !xs || !wq || !ws) return W4A4_E_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(xs, 4) || !aligned(ws, 4)) return W4A4_E_ALIGN;
  g.a = xq; g.sa = xs; g.w = wq; g.sw = ws;
  g.ga = ga; g.gw = gw;
  g.M = M; g.N = N; g.K = K;
  return W4A4_OK;
}

w4a4_status_t w4a4_gemm(const uint8_t* xq, const float* xs, int32_t group_a,
                        const uint8_t* wq, const float* ws, int32_t group_w,
                        int64_t M, int64_t N, int64_t K,
                        void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = gemm_common(xq, xs, group_a, wq, ws, group_w, M, N, K, g);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if ((st = check_y(y, y_dtype, N, ldy)) != W4A4_OK) return st;
  g.y = y; g.ydtype = y_dtype; g.ldy = ldy;
  g.m0 = 0; g.mc = M; g.n0 = 0; g.nc = N; g.partials = nullptr;
  w4a4::launch_w4a4_gemm(g, as_stream(stream));
  return launched();
}

int64_t w4a4_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w,
                                   int32_t splits) {
  if (M < 0 || N < 0 || K <= 0 || K % 128 || K > kMaxGemmK || splits < 0) return -1;
  if (!gemm_groups_ok(K, group_a, group_w)) return -1;
  if (M == 0 || N == 0) return 0;
  const w4a4::SplitPlan pl = w4a4::plan_w4a4_splitk(M, N, K, group_a, group_w, splits);
  return pl.splits > 1 ? (int64_t)pl.splits * M * N * 4 : 0;
}

w4a4_status_t w4a4_gemm_splitk(const uint8_t* xq, const float* xs, int32_t group_a,
                               const uint8_t* wq, const float* ws, int32_t group_w,
                               int64_t M, int64_t N, int64_t K, int32_t splits,
                               void* workspace, int64_t workspace_bytes,
                               void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = gemm_common(xq, xs, group_a, wq, ws, group_w, M, N, K, g);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if (splits < 0) return W4A4_E_SHAPE;
  if ((st = check_y(y, y_dtype, N, ldy)) != W4A4_OK) return st;
  g.y = y; g.ydtype = y_dtype; g.ldy = ldy;
  g.m0 = 0; g.mc = M; g.n0 = 0; g.nc = N; g.partials = nullptr;
  const w4a4::SplitPlan pl = w4a4::plan_w4a4_splitk(M, N, K, group_a, group_w, splits);
  if (pl.splits == 1) {
    w4a4::launch_w4a4_gemm(g, as_stream(stream));
    return launched();
  }
  if (workspace_bytes < (int64_t)pl.splits * M * N * 4) return W4A4_E_SHAPE;
  if (!workspace) return W4A4_E_NULL;
  if (!aligned(workspace, 16)) return W4A4_E_ALIGN;
  w4a4::launch_w4a4_gemm_splitk(g, pl, static_cast<float*>(workspace), as_stream(stream));
  return launched();
}

w4a4_status_t w4a4_gemm_debug_partials(const uint8_t* xq, const float* xs, int32_t group_a,
                                       const uint8_t* wq, const float* ws, int32_t group_w,
                                       int64_t M, int64_t N, int64_t K,
                                       int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                       int32_t* partials, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = gemm_common(xq, xs, group_a, wq, ws, group_w, M, N, K, g);
  if (st != W4A4_OK) return st;
  if ((st = check_window(M, N, m0, mc, n0, nc)) != W4A4_OK) return st;
  if (!partials) return W4A4_E_NULL;
  if (!aligned(partials, 4)) return W4A4_E_ALIGN;
  g.y = nullptr; g.ydtype = 0; g.ldy = 0;
  g.m0 = m0; g.mc = mc; g.n0 = n0; g.nc = nc; g.partials = partials;
  w4a4::launch_w4a4_gemm(g, as_stream(stream));
  return launched();
}

static w4a4_status_t mx_quant(const void* x, int64_t rows, int64_t K, int64_t ldx,
                              uint8_t* q, uint8_t* e8m0, int mode, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 || ldx < K) return W4A4_E_SHAPE;
  if (ldx % 8) return W4A4_E_ALIGN;
  if (rows == 0) return W4A4_OK;
  if (!x || !q || !e8m0) return W4A4_E_NULL;
  if (!aligned(x, 16) || !aligned(q, 4)) return W4A4_E_ALIGN;
  w4a4::launch_mxfp4_quant(x, rows, K, ldx, q, e8m0, mode, as_stream(stream));
  return launched();
}

w4a4_status_t mxfp4_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx,
                             uint8_t* q, uint8_t* e8m0, void* stream) {
  return mx_quant(x, rows, K, ldx, q, e8m0, 0, stream);
}

w4a4_status_t mxfp4_quantize_residual(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                      uint8_t* q, uint8_t* e8m0, void* stream) {
  return mx_quant(x, rows, K, ldx, q, e8m0, 1, stream);
}

w4a4_status_t mxfp4_quantize_residual_tied(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                           uint8_t* q, uint8_t* e8m0, void* stream) {
  return mx_quant(x, rows, K, ldx, q, e8m0, 3, stream);
}

w4a4_status_t mxfp4_quantize_append_copy(const void* w, int64_t rows, int64_t K, int64_t ldw,
                                         uint8_t* q, uint8_t* e8m0, void* stream) {
  return mx_quant(w, rows, K, ldw, q, e8m0, 2, stream);
}

static w4a4_status_t mx_common(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                               int64_t M, int64_t N, int64_t K, GemmArgs& g) {
  // K <= 2^23: a 256-row tile then spans < 2^31 bytes, the kernel's 32-bit
  // buffer offsets
  if (M < 0 || N < 0 || K <= 0 || K % 128 || K > (int64_t{1} << 23)) return W4A4_E_SHAPE;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!xq || !xe || !wq || !we) return W4A4_E_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(xe, 4) || !aligned(we, 4)) return W4A4_E_ALIGN;
  g.a = xq; g.sa = xe; g.w = wq; g.sw = we;
  g.ga = 32; g.gw = 32;
  g.M = M; g.N = N; g.K = K;
  return W4A4_OK;
}

w4a4_status_t mxfp4_gemm(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                         int64_t M, int64_t N, int64_t K,
                         void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = mx_common(xq, xe, wq, we, M, N, K, g);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if ((st = check_y(y, y_dtype, N, ldy)) != W4A4_OK) return st;
  g.y = y; g.ydtype = y_dtype; g.ldy = ldy;
  g.m0 = 0; g.mc = M; g.n0 = 0; g.nc = N; g.partials = nullptr;
  w4a4::launch_mxfp4_gemm(g, as_stream(stream));
  return launched();
}

w4a4_status_t mxfp4_gemm_debug_partials(const uint8_t* xq, const uint8_t* xe,
                                        const uint8_t* wq, const uint8_t* we,
                                        int64_t M, int64_t N, int64_t K,
                                        int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                        int32_t* partials, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = mx_common(xq, xe, wq, we, M, N, K, g);
  if (st != W4A4_OK) return st;
  if ((st = check_window(M, N, m0, mc, n0, nc)) != W4A4_OK) return st;
  if (!partials) return W4A4_E_NULL;
  if (!aligned(partials, 4)) return W4A4_E_ALIGN;
  g.y = nullptr; g.ydtype = 0; g.ldy = 0;
  g.m0 = m0; g.mc = mc; g.n0 = n0; g.nc = nc; g.partials = partials;
  w4a4::launch_mxfp4_gemm(g, as_stream(stream));
  return launched();
}

static w4a4_status_t nv_quant_shape(int64_t rows, int64_t K, int64_t ldx) {
  if (rows < 0 || K <= 0 || K % 256 || ldx < K || K > (int64_t{1} << 30)) return W4A4_E_SHAPE;
  if (ldx % 8) return W4A4_E_ALIGN;
  return W4A4_OK;
}

w4a4_status_t nvfp4_global_scale(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                 float* global_scale, void* stream) {
  if (rows < 0 || K <= 0 || K % 8 || ldx < K || K > (int64_t{1} << 30)) return W4A4_E_SHAPE;
  if (ldx % 8) return W4A4_E_ALIGN;
  if (!global_scale || (rows > 0 && !x)) return W4A4_E_NULL;
  if (!aligned(global_scale, 4) || (rows > 0 && !aligned(x, 16))) return W4A4_E_ALIGN;
  w4a4::launch_nvfp4_global_scale(x, rows, K, ldx, global_scale, as_stream(stream));
  return launched();
}

w4a4_status_t nvfp4_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx, const float* global_scale,
                             uint8_t* q, uint8_t* scales, void* stream) {
  w4a4_status_t st = nv_quant_shape(rows, K, ldx);
  if (st != W4A4_OK || rows == 0) return st;
  if (!x || !global_scale || !q || !scales) return W4A4_E_NULL;
  if (!aligned(x, 16) || !aligned(global_scale, 4) || !aligned(q, 4) || !aligned(scales, 2)) return W4A4_E_ALIGN;
  w4a4::launch_nvfp4_quant(x, rows, K, ldx, global_scale, q, scales, as_stream(stream));
  return launched();
}

static w4a4_status_t nv_common(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws,
                               int64_t M, int64_t N, int64_t K, GemmArgs& g) {
  // K <= 2^23: a 256-row tile then spans < 2^31 bytes, the kernel's 32-bit
  // buffer offsets
  if (M < 0 || N < 0 || K <= 0 || K % 256 || K > (int64_t{1} << 23)) return W4A4_E_SHAPE;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!xq || !xs || !wq || !ws) return W4A4_E_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(xs, 16) || !aligned(ws, 16)) return W4A4_E_ALIGN;
  g.a = xq; g.sa = xs; g.w = wq; g.sw = ws;
  g.ga = 16; g.gw = 16;
  g.M = M; g.N = N; g.K = K;
  return W4A4_OK;
}

w4a4_status_t nvfp4_gemm(const uint8_t* xq, const uint8_t* xs, const float* x_global,
                         const uint8_t* wq, const uint8_t* ws, const float* w_global,
                         int64_t M, int64_t N, int64_t K,
                         void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = nv_common(xq, xs, wq, ws, M, N, K, g);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if (!x_global || !w_global) return W4A4_E_NULL;
  if (!aligned(x_global, 4) || !aligned(w_global, 4)) return W4A4_E_ALIGN;
  if ((st = check_y(y, y_dtype, N, ldy)) != W4A4_OK) return st;
  g.y = y; g.ydtype = y_dtype; g.ldy = ldy;
  g.m0 = 0; g.mc = M; g.n0 = 0; g.nc = N; g.partials = nullptr;
  w4a4::launch_nvfp4_gemm(g, x_global, w_global, as_stream(stream));
  return launched();
}

w4a4_status_t nvfp4_gemm_debug_partials(const uint8_t* xq, const uint8_t* xs,
                                        const uint8_t* wq, const uint8_t* ws,
                                        int64_t M, int64_t N, int64_t K,
                                        int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                        int32_t* partials, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = nv_common(xq, xs, wq, ws, M, N, K, g);
  if (st != W4A4_OK) return st;
  if ((st = check_window(M, N, m0, mc, n0, nc)) != W4A4_OK) return st;
  if (!partials) return W4A4_E_NULL;
  if (!aligned(partials, 4)) return W4A4_E_ALIGN;
  g.y = nullptr; g.ydtype = 0; g.ldy = 0;
  g.m0 = m0; g.mc = mc; g.n0 = n0; g.nc = nc; g.partials = partials;
  w4a4::launch_nvfp4_gemm(g, nullptr, nullptr, as_stream(stream));
  return launched();
}

// -------------------------------------------------------- fused decode path

int32_t w4a4_linear_fused_supported(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w) {
  if (M < 1 || N < 1 || K <= 0 || K % 128 || K > kMaxGemmK) return 0;
  if (!gemm_groups_ok(K, group_a, group_w)) return 0;
  return w4a4::linear_small_supported(M, N, K, group_a, group_w) ? 1 : 0;
}

w4a4_status_t w4a4_linear_fused(const void* x, int64_t M, int64_t K, int64_t ldx, int32_t group_a,
                                const uint8_t* wq, const float* ws, int32_t group_w, int64_t N,
                                void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 128 || K > kMaxGemmK || ldx < K) return W4A4_E_SHAPE;
  if (!gemm_groups_ok(K, group_a, group_w)) return W4A4_E_GROUP;
  if (ldx % 8) return W4A4_E_ALIGN;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!w4a4_linear_fused_supported(M, N, K, group_a, group_w)) return W4A4_E_SHAPE;
  w4a4_status_t st = check_y(y, y_dtype, N, ldy);
  if (st != W4A4_OK) return st;
  if (!x || !wq || !ws) return W4A4_E_NULL;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(ws, 4)) return W4A4_E_ALIGN;
  w4a4::launch_w4a4_linear_small(x, M, K, ldx, group_a, wq, ws, group_w, N, y, y_dtype, ldy, as_stream(stream));
  return launched();
}

// ------------------------------------------------------ no-allocation split-K
}  // extern "C"

namespace {

// Split-K partial outputs of w4a4_gemm_splitk_noalloc: a file-scope device
// array, one copy per GPU, alive until the process ends. Its name is a host
// stand-in, not a device address: host code only ever uses the address that
// hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchBytes = int64_t{32} << 20;
static __device__ __align__(256) float scratch[kScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device), or
// nullptr when the runtime reports an error.
float* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int64_t w4a4_gemm_splitk_noalloc_max_bytes(void) { return kScratchBytes; }

w4a4_status_t w4a4_gemm_splitk_noalloc(const uint8_t* xq, const float* xs, int32_t group_a,
                                       const uint8_t* wq, const float* ws, int32_t group_w,
                                       int64_t M, int64_t N, int64_t K, int32_t splits,
                                       void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  GemmArgs g = {};
  w4a4_status_t st = gemm_common(xq, xs, group_a, wq, ws, group_w, M, N, K, g);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if (splits < 0) return W4A4_E_SHAPE;
  if ((st = check_y(y, y_dtype, N, ldy)) != W4A4_OK) return st;
  g.y = y; g.ydtype = y_dtype; g.ldy = ldy;
  g.m0 = 0; g.mc = M; g.n0 = 0; g.nc = N; g.partials = nullptr;
  const w4a4::SplitPlan pl = w4a4::plan_w4a4_splitk(M, N, K, group_a, group_w, splits);
  if (pl.splits == 1) {
    w4a4::launch_w4a4_gemm(g, as_stream(stream));
    return launched();
  }
  // every split writes its whole [M][N] partial output: nothing needs clearing
  if ((int64_t)pl.splits * M * N * 4 > kScratchBytes) return W4A4_E_SCRATCH;
  float* ws_dev = device_scratch();
  if (!ws_dev) return W4A4_E_HIP;
  w4a4::launch_w4a4_gemm_splitk(g, pl, ws_dev, as_stream(stream));
  return launched();
}

// ---------------------------------------------------------- storage conversions

w4a4_status_t w4a4_repack_int4(const uint8_t* nibbles, int64_t rows, int64_t K, uint8_t* packed,
                               int32_t* minus8_count, void* stream) {
  if (rows < 0 || K <= 0 || K % 16) return W4A4_E_SHAPE;
  if (rows == 0) {
    if (minus8_count) w4a4::launch_repack_int4(nullptr, 0, K, nullptr, minus8_count, as_stream(stream));
    return minus8_count ? launched() : W4A4_OK;
  }
  if (!nibbles || !packed) return W4A4_E_NULL;
  if (!aligned(nibbles, 8) || !aligned(packed, 8) || (minus8_count && !aligned(minus8_count, 4))) return W4A4_E_ALIGN;
  w4a4::launch_repack_int4(nibbles, rows, K, packed, minus8_count, as_stream(stream));
  return launched();
}

w4a4_status_t w4a4_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, uint8_t* nibbles, void* stream) {
  if (rows < 0 || K <= 0 || K % 16) return W4A4_E_SHAPE;
  if (rows == 0) return W4A4_OK;
  if (!nibbles || !packed) return W4A4_E_NULL;
  if (!aligned(nibbles, 8) || !aligned(packed, 8)) return W4A4_E_ALIGN;
  w4a4::launch_unpack_int4(packed, rows, K, nibbles, as_stream(stream));
  return launched();
}

// [rows][cols] -> [cols][rows]; the grid's second dimension covers 32 rows per block
static w4a4_status_t transpose_scales(const float* in, int64_t rows, int64_t cols, float* out, void* stream) {
  if (rows < 0 || cols < 0 || rows > 65535LL * 32 || cols > (int64_t{1} << 31)) return W4A4_E_SHAPE;
  if (rows == 0 || cols == 0) return W4A4_OK;
  if (!in || !out) return W4A4_E_NULL;
  if (!aligned(in, 4) || !aligned(out, 4)) return W4A4_E_ALIGN;
  w4a4::launch_transpose_f32(in, rows, cols, out, as_stream(stream));
  return launched();
}

w4a4_status_t w4a4_scales_to_group_major(const float* scales_rows, int64_t rows, int64_t groups,
                                         float* scales_gm, void* stream) {
  return transpose_scales(scales_rows, rows, groups, scales_gm, stream);
}

w4a4_status_t w4a4_scales_to_row_major(const float* scales_gm, int64_t rows, int64_t groups,
                                       float* scales_rows, void* stream) {
  return transpose_scales(scales_gm, groups, rows, scales_rows, stream);
}

static w4a4_status_t scale_panels(int fmt, bool to_panels, const uint8_t* in, int64_t rows, int64_t K,
                                  int64_t kmul, uint8_t* out, void* stream) {
  if (rows < 0 || K <= 0 || K % kmul) return W4A4_E_SHAPE;
  if (rows == 0) return W4A4_OK;
  if (!in || !out) return W4A4_E_NULL;
  w4a4::launch_scale_panels(fmt, to_panels, in, rows, K / (fmt == 0 ? 32 : 16), out, as_stream(stream));
  return launched();
}

w4a4_status_t mxfp4_scales_to_panels(const uint8_t* e8m0_rows, int64_t rows, int64_t K, uint8_t* e8m0,
                                     void* stream) {
  return scale_panels(0, true, e8m0_rows, rows, K, 32, e8m0, stream);
}

w4a4_status_t mxfp4_scales_to_rows(const uint8_t* e8m0, int64_t rows, int64_t K, uint8_t* e8m0_rows,
                                   void* stream) {
  return scale_panels(0, false, e8m0, rows, K, 32, e8m0_rows, stream);
}

w4a4_status_t nvfp4_scales_to_panels(const uint8_t* scales_rows, int64_t rows, int64_t K, uint8_t* scales,
                                     void* stream) {
  return scale_panels(1, true, scales_rows, rows, K, 256, scales, stream);
}

w4a4_status_t nvfp4_scales_to_rows(const uint8_t* scales, int64_t rows, int64_t K, uint8_t* scales_rows,
                                   void* stream) {
  return scale_panels(1, false, scales, rows, K, 256, scales_rows, stream);
}

}  // extern "C"
