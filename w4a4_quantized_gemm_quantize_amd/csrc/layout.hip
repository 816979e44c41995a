// Conversions between the canonical storage of codes and scales and the
// layouts the GEMMs read (gfx950). The pages fix no storage layout; the
// canonical forms are the plain ones a caller holding INT4 / MXFP4 / NVFP4
// data from elsewhere has: two's-complement nibbles with the even k in the
// low nibble, and row-major scales [rows][K / block]. The GEMM layouts (see
// the C header) exist for the matrix cores and the L2 request count; these
// kernels move data between the two without changing a value, so a model
// packed elsewhere can be fed to the GEMMs ("drop-in" use, APEX4 abstract).
// All are memory-bound byte permutations: one pass over the bytes.
#include "device.h"
#include "launch.h"

namespace w4a4 {

namespace {

// Folding masks of the GEMM's INT4 unit: X holds stream word S0 plus, at bit
// positions 3, 4 mod 6, bits of S1; Y holds S2 plus, at 0, 5 mod 6, the rest of S1.
constexpr uint32_t kFoldX = 0x18618618u;
constexpr uint32_t kFoldY = 0x61861861u;

// 16 two's-complement nibbles (lo: codes 0..7, hi: codes 8..15, even code in
// the low nibble of each byte) -> the GEMM unit X, Y. Field k of the 96-bit
// stream (bits 6k .. 6k+5) is sign << 5 | magnitude. A code -8 has no
// sign-magnitude form in 4 bits of magnitude 0..7: it is stored as +0 and
// counted in *bad.
__device__ __forceinline__ uint2 fold16(uint32_t lo, uint32_t hi, int& bad) {
  uint32_t s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t nib = ((k < 8 ? lo : hi) >> (4 * (k & 7))) & 15u;
    const int c = nib >= 8 ? (int)nib - 16 : (int)nib;
    uint32_t f = 0;
    if (c == -8)
      ++bad;
    else
      f = (c < 0 ? 32u : 0u) | (uint32_t)(c < 0 ? -c : c);
    const int p = 6 * k, d = p >> 5, off = p & 31;
    const uint32_t part = f << off;
    const uint32_t spill = off > 26 ? f >> (32 - off) : 0u;
    if (d == 0) {
      s0 |= part;
      s1 |= spill;
    } else if (d == 1) {
      s1 |= part;
      s2 |= spill;
    } else {
      s2 |= part;
    }
  }
  return uint2{s0 | (s1 & kFoldX), s2 | (s1 & kFoldY)};
}

// The inverse: GEMM unit X, Y -> 16 two's-complement nibbles (a stored -0 becomes 0).
__device__ __forceinline__ uint2 unfold16(uint32_t x, uint32_t y) {
  const uint32_t s[3] = {x & ~kFoldX, (x & kFoldX) | (y & kFoldY), y & ~kFoldY};
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int p = 6 * k, d = p >> 5, off = p & 31;
    uint32_t f = s[d] >> off;
    if (off > 26) f |= s[d + 1] << (32 - off);
    const int mag = (int)(f & 7u);
    const int c = (f & 32u) ? -mag : mag;
    const uint32_t nib = (uint32_t)c & 15u;
    if (k < 8)
      lo |= nib << (4 * k);
    else
      hi |= nib << (4 * (k - 8));
  }
  return uint2{lo, hi};
}

__global__ void k_clear_count(int32_t* count) { *count = 0; }

// One 8-byte unit (16 codes) per thread, grid-stride; both arrays are
// contiguous [rows][K/2] and 8-byte aligned, so unit u sits at byte 8u in both.
__global__ __launch_bounds__(256) void k_repack_int4(const uint2* __restrict__ in, int64_t units,
                                                    uint2* __restrict__ out, int32_t* __restrict__ count) {
  int bad = 0;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += (int64_t)gridDim.x * blockDim.x) {
    const uint2 v = in[u];
    out[u] = fold16(v.x, v.y, bad);
  }
  if (count) {
    // wave total of the -8 codes, one atomic per wave that saw any
    const unsigned long long any = __ballot(bad != 0);
    if (any) {
      int total = bad;
      for (int s = 32; s > 0; s >>= 1) total += __shfl_xor(total, s);
      if ((threadIdx.x & 63) == __ffsll((long long)any) - 1) atomicAdd(count, total);
    }
  }
}

__global__ __launch_bounds__(256) void k_unpack_int4(const uint2* __restrict__ in, int64_t units,
                                                    uint2* __restrict__ out) {
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += (int64_t)gridDim.x * blockDim.x) {
    const uint2 v = in[u];
    out[u] = unfold16(v.x, v.y);
  }
}

// out[c][r] = in[r][c] for a [rows][cols] fp32 matrix, through a 32 x 33 LDS
// tile so both the reads and the writes are row-contiguous.
__global__ __launch_bounds__(256) void k_transpose_f32(const float* __restrict__ in, int64_t rows, int64_t cols,
                                                      float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int64_t c0 = (int64_t)blockIdx.x * 32, r0 = (int64_t)blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8 threads
  for (int j = ty; j < 32; j += 8) {
    const int64_t r = r0 + j, c = c0 + tx;
    if (r < rows && c < cols) tile[j][tx] = in[r * cols + c];
  }
  __syncthreads();
  for (int j = ty; j < 32; j += 8) {
    const int64_t c = c0 + j, r = r0 + tx;
    if (r < rows && c < cols) out[c * rows + r] = tile[tx][j];
  }
}

// Byte offset of the scale of (row r, block b) in the 256-k panel layouts.
// E8M0 (blocks of 32): panel p = b / 8 holds w_p = min(8, nb - 8p) bytes per
// row, row after row, even blocks of the panel first.
__device__ __forceinline__ int64_t e8m0_offset(int64_t rows, int64_t nb, int64_t r, int64_t b) {
  const int64_t p = b >> 3, j = b & 7;
  const int64_t w = nb - 8 * p < 8 ? nb - 8 * p : 8;
  const int64_t pos = (j & 1) ? (w + 1) / 2 + j / 2 : j / 2;
  return 8 * rows * p + w * r + pos;
}

// E4M3 (blocks of 16): panel p = b / 16 holds 16 bytes per row, row after
// row, blocks 0,1,4,5,8,9,12,13 then 2,3,6,7,10,11,14,15.
__device__ __forceinline__ int64_t e4m3_offset(int64_t rows, int64_t r, int64_t b) {
  const int64_t p = b >> 4, j = b & 15;
  return 16 * rows * p + 16 * r + 8 * ((j >> 1) & 1) + 2 * (j >> 2) + (j & 1);
}

// One scale byte per thread: TO_PANELS moves row-major [rows][nb] into the
// panel layout, else back. FMT 0: E8M0, 1: E4M3.
template <int FMT, bool TO_PANELS>
__global__ __launch_bounds__(256) void k_scale_panels(const uint8_t* __restrict__ in, int64_t rows, int64_t nb,
                                                     uint8_t* __restrict__ out) {
  const int64_t n = rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nb, b = i - r * nb;
    const int64_t off = FMT == 0 ? e8m0_offset(rows, nb, r, b) : e4m3_offset(rows, r, b);
    if (TO_PANELS)
      out[off] = in[i];
    else
      out[i] = in[off];
  }
}

unsigned grid_for(int64_t items) {
  const int64_t blocks = (items + 255) / 256;
  return (unsigned)(blocks < 16384 ? (blocks > 0 ? blocks : 1) : 16384);
}

}  // namespace

void launch_repack_int4(const uint8_t* nibbles, int64_t rows, int64_t K, uint8_t* packed, int32_t* count,
                        hipStream_t stream) {
  const int64_t units = rows * K / 16;
  if (count) hipLaunchKernelGGL(k_clear_count, dim3(1), dim3(1), 0, stream, count);
  hipLaunchKernelGGL(k_repack_int4, dim3(grid_for(units)), dim3(256), 0, stream,
                     reinterpret_cast<const uint2*>(nibbles), units, reinterpret_cast<uint2*>(packed), count);
}

void launch_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, uint8_t* nibbles, hipStream_t stream) {
  const int64_t units = rows * K / 16;
  hipLaunchKernelGGL(k_unpack_int4, dim3(grid_for(units)), dim3(256), 0, stream,
                     reinterpret_cast<const uint2*>(packed), units, reinterpret_cast<uint2*>(nibbles));
}

void launch_transpose_f32(const float* in, int64_t rows, int64_t cols, float* out, hipStream_t stream) {
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL(k_transpose_f32, grid, dim3(256), 0, stream, in, rows, cols, out);
}

void launch_scale_panels(int fmt, bool to_panels, const uint8_t* in, int64_t rows, int64_t nb, uint8_t* out,
                         hipStream_t stream) {
  const dim3 grid(grid_for(rows * nb));
  if (fmt == 0) {
    if (to_panels)
      hipLaunchKernelGGL((k_scale_panels<0, true>), grid, dim3(256), 0, stream, in, rows, nb, out);
    else
      hipLaunchKernelGGL((k_scale_panels<0, false>), grid, dim3(256), 0, stream, in, rows, nb, out);
  } else {
    if (to_panels)
      hipLaunchKernelGGL((k_scale_panels<1, true>), grid, dim3(256), 0, stream, in, rows, nb, out);
    else
      hipLaunchKernelGGL((k_scale_panels<1, false>), grid, dim3(256), 0, stream, in, rows, nb, out);
  }
}

}  // namespace w4a4
