/*
 * w4a4.h -- C ABI of libw4a4.so: W4A4 group-quantized GEMM, MXFP4 GEMM and
 * NVFP4 GEMM on AMD Instinct MI355X (gfx950).
 *
 * What is computed (see the operation comments below for the passages):
 *   Y[M,N] = X[M,K] * W[N,K]^T for a linear layer whose activations X and
 *   weights W are both 4-bit ("W4A4"), either
 *   - INT4 with one fp32 scale per group of g consecutive K elements
 *     ("APEX4: Efficient Pure W4A4 LLM Inference via Intra-SM Compute
 *     Rebalancing", abstract: the W4A4-g128 pure INT4 GEMM whose per-group
 *     dequantization runs on the vector units, and its mixed-granularity mode),
 *   - or MXFP4: FP4 E2M1 values with one E8M0 power-of-two scale per 32 K
 *     elements ("the open-standard MXFP4", FP4 RL post-training abstract on the
 *     "Depth Registers Unlock W4A4 on SwiGLU" page; block rule from the OCP
 *     Microscaling Formats v1.0 specification),
 *   - or NVFP4: FP4 E2M1 values with one FP8 E4M3 scale per 16 K elements and
 *     one binary32 global scale per tensor (ARCQuant abstract on the APEX4
 *     page; Minima abstract on the "Daily Papers" page: 16-element block
 *     scaling and a calibrated per-module global scale).
 *
 * Conventions (all entry points):
 *   - Every data pointer is a DEVICE pointer, owned by the caller. The library
 *     allocates no memory and keeps no mutable state; it is thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous on that stream; nothing synchronizes.
 *   - Arguments are validated first, synchronously, before any HIP call. On a
 *     validation failure the call returns the status and launches nothing.
 *     A launch failure reported by hipGetLastError() returns W4A4_E_HIP.
 *   - Extents are int64_t element counts. A zero extent (M, N or rows == 0) is a
 *     valid no-op; pointers whose extent is zero may then be NULL.
 *   - Buffers must not overlap. Results are deterministic (no floating-point
 *     atomics; nvfp4_global_scale's one integer atomic max is order-free).
 *   - Packed 4-bit codes are row-major [rows][K/2] bytes, K contiguous, 4 bits
 *     per code.
 *     MXFP4 and NVFP4: E2M1 codes (sign<<3 | magnitude index into
 *     {0,0.5,1,1.5,2,3,4,6}), two per byte, the even k in the LOW nibble.
 *     INT4: sign-magnitude (the symmetric rule below only yields codes in
 *     [-7, 7]), the sign bit being that of the input value (a negative input
 *     that rounds to 0 is stored as -0). Each 8-byte unit holds the codes
 *     c0..c15 of 16 consecutive k as two little-endian 32-bit words X, Y. Let
 *     S be the 96-bit stream with the 6-bit field f_k = sign_k << 5 | |c_k| at
 *     bits 6k..6k+5 -- the OCP FP6 E2M3 encoding of the subnormal +-|c_k|/8,
 *     whose bits 3 and 4 are always zero -- and S0, S1, S2 its 32-bit words:
 *       X = S0 | (S1 & 0x18618618),   Y = S2 | (S1 & 0x61861861)
 *     (0x18618618 marks bit positions 3, 4 mod 6, where S0 is zero;
 *     0x61861861 marks 0, 5 mod 6, where S2 is zero). The GEMM rebuilds its
 *     FP6 operand as S0 = X & 0xE79E79E7, S1 = (X & 0x18618618) |
 *     (Y & 0x61861861), S2 = Y & 0x9E79E79E; the matrix cores then multiply
 *     the codes exactly (E8M0 scale 2^3 per operand).
 */
#ifndef W4A4_H
#define W4A4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A4_OK = 0,
  W4A4_E_NULL = 1,   /* a required pointer is NULL */
  W4A4_E_SHAPE = 2,  /* negative extent, K not a supported multiple, ld too small, or window out of range */
  W4A4_E_GROUP = 3,  /* unsupported group size, group does not divide K, or groups do not nest */
  W4A4_E_ALIGN = 4,  /* a pointer or leading dimension breaks the alignment rule of the call */
  W4A4_E_DTYPE = 5,  /* unknown output dtype */
  W4A4_E_HIP = 6,    /* the HIP runtime reported an error for the launch */
  W4A4_E_SCRATCH = 7 /* the call needs more than the library's static scratch buffer */
} w4a4_status_t;

typedef enum {
  W4A4_Y_F32 = 0,    /* fp32 output */
  W4A4_Y_F16 = 1     /* fp16 output, round to nearest even from the fp32 result */
} w4a4_ydtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* w4a4_status_str(int status);

/*
 * Symmetric INT4 quantization of activations, per row, in groups of `group`
 * consecutive K elements (APEX4 abstract: W4A4-g128, activations quantized to
 * 4 bits per group of 128; other group sizes serve its mixed-granularity mode).
 * Per group: a = max|x|; s = fl32(a / 7); q = clamp(rne(fl32(x / s)), -8, 7)
 * with correctly rounded binary32 divisions; an all-zero group gives s = 0 and
 * codes 0. (The pages give no formula: this is the plain symmetric reading.)
 * |x| <= a makes |q| <= 7, so the codes fit the sign-magnitude layout above.
 *
 *   x     fp16 [M][ldx] row-major, 16-byte aligned, ldx >= K, ldx % 8 == 0
 *   M, K  K > 0, K % 16 == 0 (K % group == 0 required as well)
 *   group 64, 128, 256, 512, or group == K ("per token")
 *   xq    out: u8 [M][K/2] packed codes (layout above), 8-byte aligned
 *   xs    out: f32 [K/group][M] scales, group-major (the scale of row m and
 *         group c is xs[c * M + m]), 4-byte aligned. One K stage of a GEMM tile
 *         then reads its rows' scales as one contiguous run.
 */
w4a4_status_t w4a4_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, int32_t group,
                                uint8_t* xq, float* xs, void* stream);

/*
 * Offline weight quantization (APEX4 abstract: 4-bit weights, "W4"): the same
 * rule as w4a4_quantize_act applied to the rows of W[N][K] (ldw = K).
 *
 *   w     fp16 [N][K], 16-byte aligned
 *   wq    out: u8 [N][K/2] (8-byte aligned);  ws  out: f32 [K/group][N] (group-major, as xs)
 */
w4a4_status_t w4a4_pack_weight(const void* w, int64_t N, int64_t K, int32_t group,
                               uint8_t* wq, float* ws, void* stream);

/*
 * W4A4 group-dequantized GEMM (APEX4 abstract: pure INT4 matrix products, with
 * the per-group dequantization -- the vector-unit bottleneck it studies -- folded
 * into the accumulation). With g = min(group_a, group_w):
 *   P_b[m,n] = sum_{k in block b of g} qa[m,k] * qw[n,k]     (exact, |P_b| <= 49 g)
 *   Y[m,n]   = sum_b s_a[m, b*g/group_a] * s_w[n, b*g/group_w] * P_b[m,n]  (fp32)
 *
 *   xq, xs          packed activation codes [M][K/2] and scales [K/group_a][M]
 *   wq, ws          packed weight codes [N][K/2] and scales [K/group_w][N]
 *                   (scales group-major, as written by the quantizers)
 *   group_a/group_w each a power of two >= 64 dividing K (64, 128, 256, 512, ...)
 *                   or K itself (per token); the larger must be a multiple of
 *                   the smaller, and g <= 262144 (P_b stays an exact integer in
 *                   the fp32 matrix-core accumulator: 49 g < 2^24)
 *   M, N, K         M, N >= 0; K > 0, K % 128 == 0 and K <= 2^23 (the kernel
 *                   addresses a 256-row tile with signed 32-bit offsets)
 *   y               out: [M][ldy] fp32 or fp16 (y_dtype), ldy >= N,
 *                   aligned to its element size
 *   xq, wq 16-byte aligned; xs, ws 4-byte aligned.
 */
w4a4_status_t w4a4_gemm(const uint8_t* xq, const float* xs, int32_t group_a,
                        const uint8_t* wq, const float* ws, int32_t group_w,
                        int64_t M, int64_t N, int64_t K,
                        void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * w4a4_gemm with K split across workgroups, for shapes whose output tiles
 * alone leave the chip's workgroup slots idle (load balancing; LLaMA-2-70B w2
 * at M = 256 has 64 tiles of 256 x 128 for 256 CUs). Split s computes the
 * group partials of its K range [s S, (s+1) S) (S whole groups' worth of
 * 128-k stages) exactly as w4a4_gemm does and writes its fp32 sum to
 * workspace[s][M][N]; a second kernel adds the splits in split order
 * (deterministic) and stores Y as y_dtype. Y differs from w4a4_gemm's only by
 * the fp32 summation order (within the same tolerance).
 *
 *   splits     0: the library picks (1 when the tiles fill the chip or the
 *              few-token path applies); > 0: at most that many (clamped to
 *              the number of groups). One split runs w4a4_gemm itself and
 *              needs no workspace.
 *   workspace  device memory of at least w4a4_gemm_splitk_workspace(...)
 *              bytes, 16-byte aligned, owned by the caller, overwritten;
 *              may be NULL when that size is 0
 *   other arguments as for w4a4_gemm.
 */
w4a4_status_t w4a4_gemm_splitk(const uint8_t* xq, const float* xs, int32_t group_a,
                               const uint8_t* wq, const float* ws, int32_t group_w,
                               int64_t M, int64_t N, int64_t K, int32_t splits,
                               void* workspace, int64_t workspace_bytes,
                               void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * Workspace bytes w4a4_gemm_splitk needs for these arguments (0 when it runs
 * unsplit), or -1 when they are invalid. Host-only; launches nothing.
 */
int64_t w4a4_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w,
                                   int32_t splits);

/*
 * Fused decode path: w4a4_quantize_act of X followed by w4a4_gemm, in ONE
 * launch, for few tokens (load balancing and launch count at decode; COMET
 * abstract on the "Daily Papers" page: fine-grained scheduling of W4A4
 * kernels). Every workgroup quantizes X itself (the same rule and arithmetic
 * as w4a4_quantize_act) into on-chip memory and runs the few-token GEMM on
 * it, so the path only serves tiny M x K; w4a4_linear_fused_supported says
 * when. Y is bit-identical to w4a4_gemm(w4a4_quantize_act(X), ...).
 *
 *   x        fp16 [M][ldx], 16-byte aligned, ldx >= K, ldx % 8 == 0
 *   group_a  64, 128, 256 or 512; group_w and wq, ws as for w4a4_gemm
 *   M, N, K  1 <= M <= 32 and 24 M K/32 + 4 M K/group_a + the cross-wave
 *            reduction buffer (3 or 7 KiB on the 16-column tiles this path
 *            takes for M <= 16 with groups >= 128; else 12 or 28 KiB) within
 *            64 KiB (LLaMA-2-70B FFN: M <= 9 for w1/w3, K = 8192; M <= 2 for
 *            w2, K = 28672); otherwise W4A4_E_SHAPE
 *   y        as for w4a4_gemm
 */
w4a4_status_t w4a4_linear_fused(const void* x, int64_t M, int64_t K, int64_t ldx, int32_t group_a,
                                const uint8_t* wq, const float* ws, int32_t group_w, int64_t N,
                                void* y, int32_t y_dtype, int64_t ldy, void* stream);

/* 1 if w4a4_linear_fused takes these extents and groups, else 0 (host-only). */
int32_t w4a4_linear_fused_supported(int64_t M, int64_t N, int64_t K, int32_t group_a, int32_t group_w);

/*
 * w4a4_gemm_splitk for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and split plan, with the splits' fp32 partial outputs in a
 * static device buffer of the library instead of a caller workspace. Calls no
 * hipMalloc, hipFree or other allocating routine.
 *   - The buffer holds w4a4_gemm_splitk_noalloc_max_bytes() bytes (32 MiB)
 *     per GPU, for the life of the process. A plan needing more
 *     (splits * M * N * 4 bytes) returns W4A4_E_SCRATCH and launches nothing;
 *     one that needs no split runs w4a4_gemm.
 *   - Every call on a GPU shares that GPU's buffer: calls that overlap on one
 *     GPU (two streams, two host threads) race and must be ordered by the
 *     caller. Each call overwrites what it uses; nothing must start at zero.
 *   - The first call on a device looks up the buffer's address there (a
 *     runtime failure returns W4A4_E_HIP).
 * Other arguments and the result are those of w4a4_gemm_splitk.
 */
w4a4_status_t w4a4_gemm_splitk_noalloc(const uint8_t* xq, const float* xs, int32_t group_a,
                                       const uint8_t* wq, const float* ws, int32_t group_w,
                                       int64_t M, int64_t N, int64_t K, int32_t splits,
                                       void* y, int32_t y_dtype, int64_t ldy, void* stream);

/* Bytes of the static buffer behind w4a4_gemm_splitk_noalloc (host-only). */
int64_t w4a4_gemm_splitk_noalloc_max_bytes(void);

/*
 * Debug export of the integer group partials P_b of w4a4_gemm for the output
 * window [m0, m0+mc) x [n0, n0+nc), from the kernel configuration w4a4_gemm
 * runs for the whole M x N x K product (same tile height or few-token path,
 * same loads, widening, matrix instructions and stage schedule; the epilogue
 * stores P_b instead of accumulating it):
 *   partials  out: int32 [K/g][mc][nc], g = min(group_a, group_w)
 * The window must lie inside [0,M) x [0,N); mc, nc > 0.
 */
w4a4_status_t w4a4_gemm_debug_partials(const uint8_t* xq, const float* xs, int32_t group_a,
                                       const uint8_t* wq, const float* ws, int32_t group_w,
                                       int64_t M, int64_t N, int64_t K,
                                       int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                       int32_t* partials, void* stream);

/*
 * MXFP4 quantization of the rows of X (OCP MX v1.0 rule; the pages name the
 * format only): per block of 32 K elements, E = floor(log2(max|x|)) - 2
 * (E = -127 for an all-zero block), scale byte E + 127, element codes =
 * E2M1(x / 2^E) rounded to nearest, ties to even, saturating at 6, sign kept.
 *
 *   x     fp16 [rows][ldx], 16-byte aligned, ldx >= K, ldx % 8 == 0; K % 32 == 0
 *   q     out: u8 [rows][K/2] packed E2M1 codes, 4-byte aligned
 *   e8m0  out: u8, rows * K/32 scale bytes in 256-k panels: with nb = K/32,
 *         w_p = min(8, nb - 8p) and j = b % 8, the scale of row r and block b
 *         (p = b / 8) is at byte 8 * rows * p + w_p * r + pos, pos = j / 2 for
 *         even j and ceil(w_p / 2) + j / 2 for odd j. Panel p thus holds, row
 *         after row, the w_p scale bytes of blocks 8p .. 8p + w_p - 1, even
 *         blocks first: a GEMM stage of 256 k reads one contiguous run per tile
 *         instead of one small piece per row, and the 4 blocks one matrix-core
 *         lane feeds sit in one dword. (K % 256 == 0: every panel is rows x 8
 *         bytes, even blocks in bytes 0..3, odd ones in 4..7.)
 * Used for activations online and for weights offline.
 */
w4a4_status_t mxfp4_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx,
                             uint8_t* q, uint8_t* e8m0, void* stream);

/*
 * Two-pass MXFP4 of the rows of X with the residual pass appended along K:
 * the activation side of the appended-residual GEMM (Multi-Scale Dequant and
 * ARCQuant abstracts, APEX4 page: the activation is split into low-precision
 * components, the residual component appended as extra reduction channels so
 * one standard block-scaled GEMM computes both terms). Output = the MXFP4
 * quantization (rule and layouts above) of the K' = 2K wide matrix
 * [x | r], where r = x - deq(Q(x)) is the exact residual of the first pass
 * and each half is quantized by the rule above with its own block scales:
 *
 *   x, K, ldx  as for mxfp4_quantize
 *   q     out: u8 [rows][K] (2K packed E2M1 codes: Q(x) then Q(r)), 4-byte aligned
 *   e8m0  out: u8, rows * 2K/32 scale bytes in the panel layout of a 2K-wide
 *         matrix (block b of Q(x) is block b, block b of Q(r) is block K/32 + b)
 *
 * mxfp4_gemm(q, e8m0, wq, we, M, N, 2K, ...) with W from
 * mxfp4_quantize_append_copy then gives Q(x) Q(w)^T + Q(r) Q(w)^T.
 */
w4a4_status_t mxfp4_quantize_residual(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                      uint8_t* q, uint8_t* e8m0, void* stream);

/*
 * Two-pass MXFP4 with the second scale tied to the first: the reading of the
 * Multi-Scale Dequant abstract (APEX4 page) under which its "error bound 1/64
 * per block" holds. Per 32-block with absmax a:
 *   first pass:  E1 = the smallest integer with a <= 6 2^E1 (so no element
 *                clips; an all-zero block takes E1 = -125), codes =
 *                E2M1(x / 2^E1) (nearest, ties to even, sign kept);
 *   second pass: r = x - deq(first) (exact), E2 = E1 - 2 (|r| <= 2^E1 keeps
 *                |r| / 2^E2 <= 4: no clipping), codes = E2M1(r / 2^E2);
 * so |x - deq(first) - deq(second)| <= 2^(E1 + 3) / 64 per element.
 * Shapes, layouts and the GEMM use as for mxfp4_quantize_residual (the first
 * pass differs from mxfp4_quantize's OCP exponent when a / 2^E would clip).
 */
w4a4_status_t mxfp4_quantize_residual_tied(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                           uint8_t* q, uint8_t* e8m0, void* stream);

/*
 * The weight side of the appended-residual GEMM: the MXFP4 quantization of
 * the rows of W written twice along K, [Q(w) | Q(w)] (shapes and layouts as
 * for mxfp4_quantize_residual, K' = 2K). Offline, like weight packing.
 */
w4a4_status_t mxfp4_quantize_append_copy(const void* w, int64_t rows, int64_t K, int64_t ldw,
                                         uint8_t* q, uint8_t* e8m0, void* stream);

/*
 * MXFP4 GEMM on the matrix cores' block-scaled FP4 path:
 *   Y[m,n] = sum_b 2^(Ea[m,b] + Ew[n,b]) * sum_{k in block b} va[m,k] * vw[n,k]
 * accumulated in fp32.
 *
 *   xq, xe   activation codes [M][K/2], M * K/32 scale bytes (panel layout
 *            of mxfp4_quantize)
 *   wq, we   weight codes [N][K/2], N * K/32 scale bytes (panel layout)
 *   K > 0, K % 128 == 0, K <= 2^23 (the kernel addresses a 256-row tile of
 *   X and W with 32-bit offsets); y as for w4a4_gemm. xq, wq 16-byte aligned.
 */
w4a4_status_t mxfp4_gemm(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                         int64_t M, int64_t N, int64_t K,
                         void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * Debug export of the exact per-block integers I_b = sum_{k in b} (2 va)(2 vw)
 * of mxfp4_gemm, from the same matrix-core instruction run one 32-block at a
 * time with unit scales, for the window [m0, m0+mc) x [n0, n0+nc):
 *   partials  out: int32 [K/32][mc][nc]
 */
w4a4_status_t mxfp4_gemm_debug_partials(const uint8_t* xq, const uint8_t* xe,
                                        const uint8_t* wq, const uint8_t* we,
                                        int64_t M, int64_t N, int64_t K,
                                        int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                        int32_t* partials, void* stream);

/*
 * NVFP4 global scale of a tensor: *global_scale = fl32(max|x| / 2688),
 * 2688 = 6 * 448 (the largest E2M1 value times the largest E4M3 value), so
 * the block holding the absmax gets the largest block scale. The pages name a
 * calibrated global scale per module (Minima abstract); this is the plain
 * choice for calibrating it from data, and for weights offline.
 *
 *   x             fp16 [rows][ldx], 16-byte aligned, ldx >= K, ldx % 8 == 0;
 *                 K % 8 == 0; finite values
 *   global_scale  out: ONE float in device memory (4-byte aligned); written on
 *                 the stream by three launches (clear, integer atomic max of
 *                 the fp16 magnitude bits, finish), so no host sync; rows == 0
 *                 writes 0.
 */
w4a4_status_t nvfp4_global_scale(const void* x, int64_t rows, int64_t K, int64_t ldx,
                                 float* global_scale, void* stream);

/*
 * NVFP4 quantization of the rows of X with a given global scale s_g (read on
 * the device from global_scale: finite, >= 0, normal or 0). Per block of 16 K
 * elements with absmax a, in correctly rounded binary32 (the pages give no
 * formula; this is the plain reading of the format):
 *   d = fl32(6 s_g); r = fl32(a / d) (a = 0: r = 0), saturated at 448;
 *   s_b = E4M3 rounding of r to nearest, ties to even (OCP FP8 E4M3FN);
 *   e = fl32(1 / fl32(s_b s_g)) (0 when that product is 0);
 *   code = E2M1 rounding of fl32(x e) to nearest, ties to even, saturating at
 *          6, the sign bit that of x (also when the magnitude rounds to 0).
 * Then x ~ v * s_b * s_g.
 *
 *   x       fp16 [rows][ldx], 16-byte aligned, ldx >= K, ldx % 8 == 0;
 *           K % 256 == 0
 *   q       out: u8 [rows][K/2] packed E2M1 codes, 4-byte aligned
 *   scales  out: u8, rows * K/16 E4M3 bytes in 256-k panels, 2-byte aligned:
 *           the scale of row r and block b (p = b / 16, j = b % 16) is at byte
 *           16 * rows * p + 16 * r + 8 * ((j >> 1) & 1) + 2 * (j >> 2) + (j & 1).
 *           A panel row thus holds blocks 0,1,4,5,8,9,12,13 in bytes 0..7 and
 *           2,3,6,7,10,11,14,15 in bytes 8..15: a GEMM stage of 256 k reads a
 *           tile's scales as one contiguous run, and each matrix-core lane the
 *           8 block scales it needs as one 8-byte word.
 */
w4a4_status_t nvfp4_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx, const float* global_scale,
                             uint8_t* q, uint8_t* scales, void* stream);

/*
 * NVFP4 GEMM: Y[m,n] = g_x g_w * sum_b s_x[m,b] s_w[n,b] * sum_{k in block b}
 * vx[m,k] vw[n,k], block b = 16 consecutive k. The matrix cores scale FP4
 * only by E8M0 powers of two per 32 elements, so each operand fragment is
 * converted to fp16 (v * s_b, exact) and multiplied on the fp16 matrix-core
 * path with fp32 accumulation; Y = fl32(acc * fl32(g_x g_w)).
 *
 *   xq, xs    activation codes [M][K/2] (16-byte aligned) and M * K/16 scale
 *             bytes (panel layout of nvfp4_quantize, 16-byte aligned)
 *   x_global  ONE float in device memory: the activations' global scale
 *   wq, ws, w_global   the same for the weights [N][K/2]
 *   K > 0, K % 256 == 0, K <= 2^23; y as for w4a4_gemm.
 */
w4a4_status_t nvfp4_gemm(const uint8_t* xq, const uint8_t* xs, const float* x_global,
                         const uint8_t* wq, const uint8_t* ws, const float* w_global,
                         int64_t M, int64_t N, int64_t K,
                         void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * Debug export of the exact per-block integers I_b = sum_{k in b} (2 vx)(2 vw)
 * of nvfp4_gemm (16-element blocks), from the same loads, conversion and
 * fp16 matrix-core instructions run one block at a time with unit scales, for
 * the window [m0, m0+mc) x [n0, n0+nc):
 *   partials  out: int32 [K/16][mc][nc]
 * The scale arrays are read (as by nvfp4_gemm) but do not enter the result.
 */
w4a4_status_t nvfp4_gemm_debug_partials(const uint8_t* xq, const uint8_t* xs,
                                        const uint8_t* wq, const uint8_t* ws,
                                        int64_t M, int64_t N, int64_t K,
                                        int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                        int32_t* partials, void* stream);

/*
 * ---- Storage conversions ------------------------------------------------
 * The pages fix no storage layout ("drop-in replacement in unmodified vLLM",
 * APEX4 abstract, asks only that a linear layer's quantized data can be fed
 * in). The canonical forms below are the plain ones: INT4 codes as
 * two's-complement nibbles, two per byte with the even k in the low nibble;
 * scales row-major [rows][K / block]. The GEMMs read the layouts documented
 * above (folded sign-magnitude INT4, group-major INT4 scales, 256-k scale
 * panels), chosen for the matrix cores and the L2 request count; these calls
 * convert on the device, value for value, in one pass over the bytes.
 * Asynchronous on `stream`, no allocation; in and out must not overlap.
 */

/*
 * Canonical INT4 codes -> the GEMM's INT4 layout.
 *   nibbles       u8 [rows][K/2] two's-complement codes in [-8, 7], even k in
 *                 the low nibble; 8-byte aligned; K % 16 == 0
 *   packed        out: u8 [rows][K/2] in the layout above, 8-byte aligned
 *   minus8_count  NULL, or ONE device int32 (4-byte aligned) that receives the
 *                 number of codes equal to -8. Those have no sign-magnitude
 *                 form in this layout (the symmetric quantizer of this
 *                 library never produces them) and are stored as 0: the
 *                 caller must check the count before using `packed`.
 */
w4a4_status_t w4a4_repack_int4(const uint8_t* nibbles, int64_t rows, int64_t K, uint8_t* packed,
                               int32_t* minus8_count, void* stream);

/*
 * The GEMM's INT4 layout -> canonical two's-complement nibbles (a stored -0
 * becomes 0). Shapes and alignment as for w4a4_repack_int4.
 */
w4a4_status_t w4a4_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, uint8_t* nibbles, void* stream);

/*
 * INT4 scales: row-major f32 [rows][groups] <-> the GEMM's group-major
 * [groups][rows] (groups = K / group size). 4-byte aligned; rows <= 2097120.
 */
w4a4_status_t w4a4_scales_to_group_major(const float* scales_rows, int64_t rows, int64_t groups,
                                         float* scales_gm, void* stream);
w4a4_status_t w4a4_scales_to_row_major(const float* scales_gm, int64_t rows, int64_t groups,
                                       float* scales_rows, void* stream);

/*
 * MXFP4 E8M0 scales: row-major u8 [rows][K/32] <-> the 256-k panel layout of
 * mxfp4_quantize (K % 32 == 0). MXFP4 codes need no conversion: the canonical
 * nibble order is the GEMM's.
 */
w4a4_status_t mxfp4_scales_to_panels(const uint8_t* e8m0_rows, int64_t rows, int64_t K, uint8_t* e8m0,
                                     void* stream);
w4a4_status_t mxfp4_scales_to_rows(const uint8_t* e8m0, int64_t rows, int64_t K, uint8_t* e8m0_rows,
                                   void* stream);

/*
 * NVFP4 E4M3 scales: row-major u8 [rows][K/16] <-> the 256-k panel layout of
 * nvfp4_quantize (K % 256 == 0).
 */
w4a4_status_t nvfp4_scales_to_panels(const uint8_t* scales_rows, int64_t rows, int64_t K, uint8_t* scales,
                                     void* stream);
w4a4_status_t nvfp4_scales_to_rows(const uint8_t* scales, int64_t rows, int64_t K, uint8_t* scales_rows,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
