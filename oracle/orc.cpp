// CPU oracle of the W4A4 group-quantized GEMM and its MXFP4 / NVFP4 variants.
//
// TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the
// benchmark's CPU-baseline leg are the only callers. The HIP library shares no
// code, header, table or helper with this file and never calls it.
//
// Plain, slow, unfused C++17, built with -O2 -ffp-contract=off (no fused
// multiply-adds, no fast-math): every binary32 step below is one correctly
// rounded IEEE operation in SSE, in the order written. Floating point that
// decides an integer (INT4 codes, NVFP4 block scales and codes) is binary32,
// the precision the GPU takes the same decision in; sums of group terms are
// binary64. Codes are plain integers (INT4: two's complement values in
// [-8, 7]; FP4: 4-bit E2M1 fields sign << 3 | index) -- no storage layout here.
// Rows are spread over std::thread workers; each output element is computed
// by one thread in a fixed order, so results do not depend on the thread count.
//
// Sources (pages cited by title and abstract; the pages give abstracts only):
//  * INT4 W4A4-g128 -- "APEX4: Efficient Pure W4A4 LLM Inference via Intra-SM
//    Compute Rebalancing", abstract: 4-bit weights and activations in groups
//    of 128 along the reduction axis, pure INT4 matrix products, per-group
//    dequantization of those products, a mixed-granularity mode. The pages give
//    no formula; the reading taken is symmetric absmax / 7 scaling, round half
//    to even, clamp to [-8, 7], binary32 scales.
//  * MXFP4 -- "the open-standard MXFP4" (FP4 RL abstract, "Depth Registers
//    Unlock W4A4 on SwiGLU" page): the OCP Microscaling Formats v1.0 block
//    rule, 32-element blocks, E8M0 scale, E2M1 elements.
//  * Two-pass MXFP4 with the residual appended along K -- Multi-Scale Dequant
//    and ARCQuant abstracts (APEX4 page).
//  * NVFP4 -- ARCQuant abstract (APEX4 page) and Minima abstract ("Daily
//    Papers" page): E2M1 elements, 16-element blocks, a calibrated global scale;
//    FP8 E4M3 block scales by the format's public definition.
#include <sched.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

// ----------------------------------------------------------------- threads

int default_threads() {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    const int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  const unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

// body(r) for every r in [0, rows), rows dealt out in contiguous chunks;
// `work` (elementary steps per row) keeps small calls on the calling thread.
void parallel_rows(int64_t rows, int threads, const std::function<void(int64_t)>& body, int64_t work = 1 << 16) {
  if (threads <= 0) threads = default_threads();
  if (rows <= 0) return;
  if (rows * work < (int64_t{1} << 18)) threads = 1;
  if (threads > rows) threads = (int)rows;
  if (threads <= 1) {
    for (int64_t r = 0; r < rows; ++r) body(r);
    return;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) {
    const int64_t r0 = rows * t / threads, r1 = rows * (t + 1) / threads;
    pool.emplace_back([r0, r1, &body] {
      for (int64_t r = r0; r < r1; ++r) body(r);
    });
  }
  for (auto& th : pool) th.join();
}

// ------------------------------------------------------ binary16 <-> binary32

uint32_t bits_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

float float_of(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// IEEE binary16 -> binary32, exact (every binary16 value is a binary32 value).
// Fields: sign 1, exponent 5 (bias 15), fraction 10.
float f16_to_f32(uint16_t h) {
  const uint32_t s = (uint32_t)(h >> 15) << 31;
  const uint32_t e = (h >> 10) & 31;
  uint32_t m = h & 1023;
  if (e == 31) return float_of(s | 0x7F800000u | (m << 13));   // infinity / NaN
  if (e == 0) {
    if (m == 0) return float_of(s);                               // signed zero
    // subnormal m * 2^-24: shift the leading one up to the hidden-bit position
    int shift = 0;
    while (!(m & 1024)) {
      m <<= 1;
      ++shift;
    }
    return float_of(s | ((uint32_t)(127 - 14 - shift) << 23) | ((m & 1023) << 13));
  }
  return float_of(s | ((e - 15 + 127) << 23) | (m << 13));
}

// IEEE binary32 -> binary16, round to nearest, ties to even; overflow gives
// infinity, NaN stays NaN (quiet).
uint16_t f32_to_f16(float f) {
  const uint32_t u = bits_of(f);
  const uint16_t s = (uint16_t)((u >> 16) & 0x8000);
  const int e = (int)((u >> 23) & 255);
  const uint32_t m = u & 0x7FFFFF;
  if (e == 255) return (uint16_t)(s | 0x7C00 | (m ? 0x200 | (m >> 13) : 0));
  if (e == 0) return s;                       // binary32 zero or subnormal: far below 2^-25
  const int E = e - 127;                      // value = sig * 2^(E - 23), sig in [2^23, 2^24)
  const uint64_t sig = (uint64_t)(m | 0x800000u);
  // target: an integer count of units u = 2^(E16 - 10), E16 = max(E, -14)
  const int E16 = E < -14 ? -14 : E;
  const int shift = 13 + (E16 - E);           // bits of sig below one unit
  if (shift > 40) return s;                   // below a quarter of the smallest subnormal
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((uint64_t{1} << shift) - 1), half = uint64_t{1} << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  // q counts units of 2^(E16-10): normal results have q in [1024, 2048]
  int ef = E < -14 ? 0 : E + 15;              // exponent field before any carry
  if (E < -14) {
    // subnormal range: q in [0, 1024]; q == 1024 is the smallest normal
    return (uint16_t)(s | q);                 // q = 1024 sets the exponent field to 1
  }
  if (q == 2048) {
    q = 1024;
    ++ef;
  }
  if (ef >= 31) return (uint16_t)(s | 0x7C00);
  return (uint16_t)(s | (ef << 10) | (q & 1023));
}

bool finite16(uint16_t h) { return ((h >> 10) & 31) != 31; }

// ------------------------------------------------------------ INT4 (APEX4)

// Per row and group of g consecutive K elements (groups start at k = 0):
//   a = max |x|                           exact
//   s = fl32(a / 7)                       binary32 division
//   q = clamp(rne(fl32(x / s)), -8, 7)    binary32 division, half to even
// An all-zero group has s = 0 and every code 0.
int int4_quantize(const uint16_t* x, int64_t R, int64_t K, int64_t g, int8_t* codes, float* scales,
                  int threads) {
  if (R < 0 || K <= 0 || g <= 0 || K % g) return 2;
  for (int64_t i = 0; i < R * K; ++i)
    if (!finite16(x[i])) return 1;
  const int64_t G = K / g;
  parallel_rows(R, threads, [&](int64_t r) {
    for (int64_t j = 0; j < G; ++j) {
      const uint16_t* xg = x + r * K + j * g;
      float a = 0.0f;
      for (int64_t k = 0; k < g; ++k) a = std::max(a, std::fabs(f16_to_f32(xg[k])));
      const float s = a / 7.0f;
      scales[r * G + j] = s;
      for (int64_t k = 0; k < g; ++k) {
        int q = 0;
        if (s != 0.0f) {
          const float t = f16_to_f32(xg[k]) / s;
          q = (int)std::nearbyint(t);   // default rounding mode: to nearest, ties to even
          q = std::min(7, std::max(-8, q));
        }
        codes[r * K + j * g + k] = (int8_t)q;
      }
    }
  }, K);
  return 0;
}

// P_b[m, n] = sum_{k in block b} qa[m, k] qw[n, k] over blocks of g along K,
// in int64; the result must fit int32 (it does for g <= 2^25: |P_b| <= 64 g).
int w4a4_block_partials(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N, int64_t K, int64_t g,
                        int32_t* P, int threads) {
  if (M < 0 || N < 0 || K <= 0 || g <= 0 || K % g) return 2;
  const int64_t B = K / g;
  std::atomic<int> overflow{0};
  parallel_rows(M, threads, [&](int64_t m) {
    for (int64_t n = 0; n < N; ++n)
      for (int64_t b = 0; b < B; ++b) {
        int64_t acc = 0;
        for (int64_t k = b * g; k < (b + 1) * g; ++k) acc += (int64_t)qa[m * K + k] * (int64_t)qw[n * K + k];
        if (acc > INT32_MAX || acc < INT32_MIN) overflow = 1;
        P[(b * M + m) * N + n] = (int32_t)acc;
      }
  }, N * K);
  return overflow ? 3 : 0;
}

// With g = min(ga, gw) (nested groups):
//   Y[m, n] = sum_b (s_a[m, b g / ga] * s_w[n, b g / gw]) * P_b[m, n]
// in binary64, block by block in b order; T is the same sum of |terms| (it
// scales the parity tolerance |Y_gpu - Y| <= 1e-5 T + 1e-6).
int w4a4_gemm(const int8_t* qa, const float* sa, int64_t ga, const int8_t* qw, const float* sw, int64_t gw,
              int64_t M, int64_t N, int64_t K, double* Y, double* T, int threads) {
  if (M < 0 || N < 0 || K <= 0 || ga <= 0 || gw <= 0 || K % ga || K % gw) return 2;
  const int64_t g = std::min(ga, gw);
  if (std::max(ga, gw) % g) return 2;
  const int64_t B = K / g, Ga = K / ga, Gw = K / gw;
  parallel_rows(M, threads, [&](int64_t m) {
    for (int64_t n = 0; n < N; ++n) {
      double y = 0.0, t = 0.0;
      for (int64_t b = 0; b < B; ++b) {
        int64_t P = 0;
        for (int64_t k = b * g; k < (b + 1) * g; ++k) P += (int64_t)qa[m * K + k] * (int64_t)qw[n * K + k];
        const double scale = (double)sa[m * Ga + b * g / ga] * (double)sw[n * Gw + b * g / gw];
        const double term = scale * (double)P;
        y += term;
        t += std::fabs(term);
      }
      Y[m * N + n] = y;
      T[m * N + n] = t;
    }
  }, N * K);
  return 0;
}

// x_hat = q s (binary64; exact: 4-bit times 24-bit significands)
void int4_dequantize(const int8_t* q, const float* s, int64_t R, int64_t K, int64_t g, double* out) {
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k) out[r * K + k] = (double)q[r * K + k] * (double)s[r * (K / g) + k / g];
}

// ------------------------------------------------------- E2M1 and MXFP4

// E2M1 magnitudes by index (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double e2m1_value(uint8_t c) { return (c & 8) ? -kE2M1[c & 7] : kE2M1[c & 7]; }

// Index of the E2M1 magnitude nearest to m >= 0, ties to the even index
// (mantissa bit 0), magnitudes beyond 6 saturating to 6. Distances are exact:
// m and the grid values have few significant bits.
int e2m1_nearest(double m) {
  if (m >= 6.0) return 7;
  int best = 0;
  double bd = m;
  for (int i = 1; i < 8; ++i) {
    const double d = std::fabs(m - kE2M1[i]);
    if (d < bd || (d == bd && (i % 2 == 0))) {
      best = i;
      bd = d;
    }
  }
  return best;
}

// The OCP MX v1.0 block rule on one block of n finite binary64 values:
//   E = floor(log2 max|v|) - 2   (2: exponent of 6, the largest E2M1 value);
//   an all-zero block takes E = -127; E is clamped to [-127, 127];
//   code = sign(v) << 3 | nearest E2M1 index of |v| 2^-E (exact scaling);
// the scale byte is E + 127.
uint8_t mx_block(const double* v, int n, uint8_t* codes) {
  double a = 0.0;
  for (int i = 0; i < n; ++i) a = std::max(a, std::fabs(v[i]));
  int E = -127;
  if (a > 0.0) {
    int ex;
    std::frexp(a, &ex);          // a = f 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    E = std::min(127, std::max(-127, ex - 1 - 2));
  }
  for (int i = 0; i < n; ++i) {
    const int idx = e2m1_nearest(std::fabs(std::ldexp(v[i], -E)));
    codes[i] = (uint8_t)((std::signbit(v[i]) ? 8 : 0) | idx);
  }
  return (uint8_t)(E + 127);
}

int mxfp4_quantize(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* e8m0, int threads) {
  if (R < 0 || K <= 0 || K % 32) return 2;
  for (int64_t i = 0; i < R * K; ++i)
    if (!finite16(x[i])) return 1;
  parallel_rows(R, threads, [&](int64_t r) {
    double v[32];
    for (int64_t b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = (double)f16_to_f32(x[r * K + b * 32 + i]);
      e8m0[r * (K / 32) + b] = mx_block(v, 32, codes + r * K + b * 32);
    }
  }, K);
  return 0;
}

// Two passes: Q(x) by the rule above, then the same rule on the exact residual
// r = x - deq(Q(x)) (binary64; r needs at most 16 significant bits) with its
// own block scales, appended along K: codes [R][2K] = [Q(x) | Q(r)], scale
// bytes [R][2K/32].
int mxfp4_quantize_residual(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* e8m0,
                            int threads) {
  if (R < 0 || K <= 0 || K % 32) return 2;
  for (int64_t i = 0; i < R * K; ++i)
    if (!finite16(x[i])) return 1;
  const int64_t nb = K / 32;
  parallel_rows(R, threads, [&](int64_t r) {
    double v[32], res[32];
    for (int64_t b = 0; b < nb; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = (double)f16_to_f32(x[r * K + b * 32 + i]);
      uint8_t* c1 = codes + r * 2 * K + b * 32;
      const uint8_t e1 = mx_block(v, 32, c1);
      e8m0[r * 2 * nb + b] = e1;
      for (int i = 0; i < 32; ++i) res[i] = v[i] - std::ldexp(e2m1_value(c1[i]), (int)e1 - 127);
      e8m0[r * 2 * nb + nb + b] = mx_block(res, 32, codes + r * 2 * K + K + b * 32);
    }
  }, K);
  return 0;
}

// Two passes with the second scale tied to the first (the reading under which
// the Multi-Scale Dequant abstract's "error bound 1/64 per block" holds): the
// first pass takes the smallest E1 with max|x| <= 6 2^E1 (nothing clips, so
// |r| <= 2^E1, half the widest E2M1 spacing), the second quantizes
// r = x - deq(Q1(x)) at the fixed scale E2 = E1 - 2 (|r| 2^-E2 <= 4: nothing
// clips), so |x - deq(Q1) - deq(Q2)| <= 2^(E1-3) = 2^(E1+3) / 64. An all-zero
// block takes E1 = -125 (bytes 2 and 0: both scales in range, codes 0).
// Layout as mxfp4_quantize_residual: [Q1(x) | Q2(r)] along K.
int mxfp4_quantize_residual_tied(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* e8m0,
                                 int threads) {
  if (R < 0 || K <= 0 || K % 32) return 2;
  for (int64_t i = 0; i < R * K; ++i)
    if (!finite16(x[i])) return 1;
  const int64_t nb = K / 32;
  parallel_rows(R, threads, [&](int64_t r) {
    for (int64_t b = 0; b < nb; ++b) {
      double v[32], a = 0.0;
      for (int i = 0; i < 32; ++i) {
        v[i] = (double)f16_to_f32(x[r * K + b * 32 + i]);
        a = std::max(a, std::fabs(v[i]));
      }
      int E1 = -125;
      if (a > 0.0) {
        E1 = -125;
        while (a > 6.0 * std::ldexp(1.0, E1)) ++E1;     // smallest E1 with a <= 6 2^E1
      }
      const int E2 = E1 - 2;
      uint8_t* c1 = codes + r * 2 * K + b * 32;
      uint8_t* c2 = codes + r * 2 * K + K + b * 32;
      for (int i = 0; i < 32; ++i) {
        c1[i] = (uint8_t)((std::signbit(v[i]) ? 8 : 0) | e2m1_nearest(std::fabs(std::ldexp(v[i], -E1))));
        const double res = v[i] - std::ldexp(e2m1_value(c1[i]), E1);
        c2[i] = (uint8_t)((std::signbit(res) ? 8 : 0) | e2m1_nearest(std::fabs(std::ldexp(res, -E2))));
      }
      e8m0[r * 2 * nb + b] = (uint8_t)(E1 + 127);
      e8m0[r * 2 * nb + nb + b] = (uint8_t)(E2 + 127);
    }
  }, K);
  return 0;
}

// x_hat = v 2^E (binary64, exact)
void mxfp4_dequantize(const uint8_t* codes, const uint8_t* e8m0, int64_t R, int64_t K, double* out) {
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k)
      out[r * K + k] = std::ldexp(e2m1_value(codes[r * K + k]), (int)e8m0[r * (K / 32) + k / 32] - 127);
}

// I_b[m, n] = sum_{k in block b} (2 va)(2 vw): 2v is an integer in [-12, 12],
// so I_b is an exact integer. Blocks of `blk` (32 for MXFP4, 16 for NVFP4).
int fp4_block_partials(const uint8_t* ca, const uint8_t* cw, int64_t M, int64_t N, int64_t K, int64_t blk,
                       int32_t* P, int threads) {
  if (M < 0 || N < 0 || K <= 0 || K % blk) return 2;
  const int64_t B = K / blk;
  parallel_rows(M, threads, [&](int64_t m) {
    for (int64_t n = 0; n < N; ++n)
      for (int64_t b = 0; b < B; ++b) {
        int64_t acc = 0;
        for (int64_t k = b * blk; k < (b + 1) * blk; ++k)
          acc += (int64_t)(2.0 * e2m1_value(ca[m * K + k])) * (int64_t)(2.0 * e2m1_value(cw[n * K + k]));
        P[(b * M + m) * N + n] = (int32_t)acc;
      }
  }, N * K);
  return 0;
}

// Y[m, n] = sum_b I_b[m, n] 2^(Ea[m, b] + Ew[n, b] - 2) in block order; each
// term is exact in binary64; T = sum of |terms|.
int mxfp4_gemm(const uint8_t* ca, const uint8_t* ea, const uint8_t* cw, const uint8_t* ew, int64_t M, int64_t N,
               int64_t K, double* Y, double* T, int threads) {
  if (M < 0 || N < 0 || K <= 0 || K % 32) return 2;
  const int64_t B = K / 32;
  parallel_rows(M, threads, [&](int64_t m) {
    for (int64_t n = 0; n < N; ++n) {
      double y = 0.0, t = 0.0;
      for (int64_t b = 0; b < B; ++b) {
        int64_t I = 0;
        for (int64_t k = b * 32; k < (b + 1) * 32; ++k)
          I += (int64_t)(2.0 * e2m1_value(ca[m * K + k])) * (int64_t)(2.0 * e2m1_value(cw[n * K + k]));
        const double term = std::ldexp((double)I, ((int)ea[m * B + b] - 127) + ((int)ew[n * B + b] - 127) - 2);
        y += term;
        t += std::fabs(term);
      }
      Y[m * N + n] = y;
      T[m * N + n] = t;
    }
  }, N * K);
  return 0;
}

// ------------------------------------------------------- E4M3 and NVFP4

// OCP FP8 E4M3 (E4M3FN): sign 1, exponent 4 (bias 7), mantissa 3; exponent
// field 0 is subnormal (m/8 2^-6); S.1111.111 is NaN; no infinities; 448 max.
double e4m3_value(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return std::nan("");
  const double mag = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

// Byte of the E4M3 value nearest to finite r in [0, 448], ties to the even
// code. Binade [2^E, 2^(E+1)) for E >= -6 holds 8 values spaced 2^(E-3); the
// subnormals below 2^-6 are spaced 2^-9. r / spacing is exact in binary64;
// rounding it half to even picks the value, and an even multiple of the
// spacing is a code with mantissa bit 0 (also across a binade edge, where the
// carry gives mantissa 0 of the next exponent).
uint8_t e4m3_round(double r) {
  int ex;
  std::frexp(r, &ex);                                  // r = f 2^ex, f in [0.5, 1)
  const int E = r > 0.0 ? std::max(ex - 1, -6) : -6;   // binade (subnormals and 0 share -6)
  const double n = std::nearbyint(std::ldexp(r, -(E - 3)));   // units of the spacing
  // value n 2^(E-3): for a normal binade n is in [8, 16] (16: carry into the next)
  int e_field, m_field;
  if (E == -6 && n < 8.0) {                            // subnormal
    e_field = 0;
    m_field = (int)n;
  } else if (n >= 16.0) {
    e_field = E + 1 + 7;
    m_field = 0;
  } else {
    e_field = E + 7;
    m_field = (int)n - 8;
  }
  return (uint8_t)(e_field * 8 + m_field);
}

// fl32(amax / 2688) with 2688 = 6 * 448 (binary32 division); 0 for no elements
int nvfp4_global_scale(const uint16_t* x, int64_t n, float* out) {
  float a = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    if (!finite16(x[i])) return 1;
    a = std::max(a, std::fabs(f16_to_f32(x[i])));
  }
  *out = a / 2688.0f;
  return 0;
}

// Per block of 16 with absmax a, in binary32:
//   d = fl32(6 s_g); r = fl32(a / d) (a = 0: r = 0) saturated at 448;
//   s_b = E4M3 rounding of r (nearest, ties to even);
//   e = fl32(1 / fl32(s_b s_g)) (0 when that product is 0);
//   code = sign(x) << 3 | nearest E2M1 index of fl32(x e) (ties to even, saturating at 6).
int nvfp4_quantize(const uint16_t* x, int64_t R, int64_t K, float sg, uint8_t* codes, uint8_t* sbytes,
                   int threads) {
  if (R < 0 || K <= 0 || K % 16) return 2;
  if (!std::isfinite(sg) || sg < 0.0f) return 4;
  for (int64_t i = 0; i < R * K; ++i)
    if (!finite16(x[i])) return 1;
  const float d = 6.0f * sg;
  parallel_rows(R, threads, [&](int64_t r) {
    for (int64_t b = 0; b < K / 16; ++b) {
      const uint16_t* xb = x + r * K + b * 16;
      float a = 0.0f;
      for (int i = 0; i < 16; ++i) a = std::max(a, std::fabs(f16_to_f32(xb[i])));
      float rr = 0.0f;
      if (a != 0.0f) rr = std::min(a / d, 448.0f);     // a / 0 = +inf saturates to 448
      const uint8_t sb = e4m3_round((double)rr);
      sbytes[r * (K / 16) + b] = sb;
      const float S = (float)e4m3_value(sb) * sg;
      const float e = S == 0.0f ? 0.0f : 1.0f / S;
      for (int i = 0; i < 16; ++i) {
        const float xv = f16_to_f32(xb[i]);
        const float t = xv * e;
        codes[r * K + b * 16 + i] = (uint8_t)((std::signbit(xv) ? 8 : 0) | e2m1_nearest(std::fabs((double)t)));
      }
    }
  }, K);
  return 0;
}

// Y[m, n] = g_a g_w sum_b (I_b (s_a[m, b] s_w[n, b])) / 4 in block order
// (binary64), the global product applied once at the end; T likewise with |terms|.
int nvfp4_gemm(const uint8_t* ca, const uint8_t* sa, float ga, const uint8_t* cw, const uint8_t* sw, float gw,
               int64_t M, int64_t N, int64_t K, double* Y, double* T, int threads) {
  if (M < 0 || N < 0 || K <= 0 || K % 16) return 2;
  const int64_t B = K / 16;
  const double G = (double)ga * (double)gw;
  parallel_rows(M, threads, [&](int64_t m) {
    for (int64_t n = 0; n < N; ++n) {
      double y = 0.0, t = 0.0;
      for (int64_t b = 0; b < B; ++b) {
        int64_t I = 0;
        for (int64_t k = b * 16; k < (b + 1) * 16; ++k)
          I += (int64_t)(2.0 * e2m1_value(ca[m * K + k])) * (int64_t)(2.0 * e2m1_value(cw[n * K + k]));
        const double term = ((double)I * (e4m3_value(sa[m * B + b]) * e4m3_value(sw[n * B + b]))) * 0.25;
        y += term;
        t += std::fabs(term);
      }
      Y[m * N + n] = y * G;
      T[m * N + n] = t * std::fabs(G);
    }
  }, N * K);
  return 0;
}

// x_hat = v s_b s_g (binary64, exact: 2 + 4 + 24 significant bits)
void nvfp4_dequantize(const uint8_t* codes, const uint8_t* sbytes, float sg, int64_t R, int64_t K, double* out) {
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k)
      out[r * K + k] = e2m1_value(codes[r * K + k]) * e4m3_value(sbytes[r * (K / 16) + k / 16]) * (double)sg;
}

}  // namespace

// ------------------------------------------------------------------ C ABI
// Status: 0 ok, 1 NaN/Inf input, 2 bad shape or group, 3 a partial does not
// fit int32, 4 bad global scale. Arrays are row-major and contiguous.
extern "C" {

int orc_default_threads() { return default_threads(); }
float orc_f16_to_f32(uint16_t h) { return f16_to_f32(h); }
uint16_t orc_f32_to_f16(float f) { return f32_to_f16(f); }

void orc_f16_to_f32_array(const uint16_t* h, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f32(h[i]);
}
void orc_f32_to_f16_array(const float* f, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16(f[i]);
}

int orc_int4_quantize(const uint16_t* x, int64_t R, int64_t K, int64_t g, int8_t* codes, float* scales,
                      int threads) {
  return int4_quantize(x, R, K, g, codes, scales, threads);
}
void orc_int4_dequantize(const int8_t* q, const float* s, int64_t R, int64_t K, int64_t g, double* out) {
  int4_dequantize(q, s, R, K, g, out);
}
int orc_w4a4_block_partials(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N, int64_t K, int64_t g,
                            int32_t* P, int threads) {
  return w4a4_block_partials(qa, qw, M, N, K, g, P, threads);
}
int orc_w4a4_gemm(const int8_t* qa, const float* sa, int64_t ga, const int8_t* qw, const float* sw, int64_t gw,
                  int64_t M, int64_t N, int64_t K, double* Y, double* T, int threads) {
  return w4a4_gemm(qa, sa, ga, qw, sw, gw, M, N, K, Y, T, threads);
}

double orc_e2m1_value(uint8_t c) { return e2m1_value(c); }
int orc_mxfp4_quantize(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* e8m0, int threads) {
  return mxfp4_quantize(x, R, K, codes, e8m0, threads);
}
int orc_mxfp4_quantize_residual(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* e8m0,
                                int threads) {
  return mxfp4_quantize_residual(x, R, K, codes, e8m0, threads);
}
int orc_mxfp4_quantize_residual_tied(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* e8m0,
                                     int threads) {
  return mxfp4_quantize_residual_tied(x, R, K, codes, e8m0, threads);
}
void orc_mxfp4_dequantize(const uint8_t* codes, const uint8_t* e8m0, int64_t R, int64_t K, double* out) {
  mxfp4_dequantize(codes, e8m0, R, K, out);
}
int orc_fp4_block_partials(const uint8_t* ca, const uint8_t* cw, int64_t M, int64_t N, int64_t K, int64_t blk,
                           int32_t* P, int threads) {
  return fp4_block_partials(ca, cw, M, N, K, blk, P, threads);
}
int orc_mxfp4_gemm(const uint8_t* ca, const uint8_t* ea, const uint8_t* cw, const uint8_t* ew, int64_t M, int64_t N,
                   int64_t K, double* Y, double* T, int threads) {
  return mxfp4_gemm(ca, ea, cw, ew, M, N, K, Y, T, threads);
}

double orc_e4m3_value(uint8_t b) { return e4m3_value(b); }
uint8_t orc_e4m3_round(double r) { return e4m3_round(r); }
int orc_nvfp4_global_scale(const uint16_t* x, int64_t n, float* out) { return nvfp4_global_scale(x, n, out); }
int orc_nvfp4_quantize(const uint16_t* x, int64_t R, int64_t K, float sg, uint8_t* codes, uint8_t* sbytes,
                       int threads) {
  return nvfp4_quantize(x, R, K, sg, codes, sbytes, threads);
}
int orc_nvfp4_gemm(const uint8_t* ca, const uint8_t* sa, float ga, const uint8_t* cw, const uint8_t* sw, float gw,
                   int64_t M, int64_t N, int64_t K, double* Y, double* T, int threads) {
  return nvfp4_gemm(ca, sa, ga, cw, sw, gw, M, N, K, Y, T, threads);
}
void orc_nvfp4_dequantize(const uint8_t* codes, const uint8_t* sbytes, float sg, int64_t R, int64_t K,
                          double* out) {
  nvfp4_dequantize(codes, sbytes, sg, R, K, out);
}

}  // extern "C"
