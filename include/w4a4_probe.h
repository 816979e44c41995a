/*
 * w4a4_probe.h -- peak probes of libw4a4.so (AMD Instinct MI355X, gfx950).
 *
 * Measurement only, not part of the W4A4 computation: loops that reach the
 * matrix-core and HBM rates of the GPU they run on, so a kernel's roofline
 * fraction can be stated against the measured peak beside the data-sheet
 * one (the pages rate kernels by measured speedups alone: APEX4 abstract).
 * Conventions as in w4a4.h: device pointers owned by the caller, asynchronous
 * on `stream`, validation first, status codes of w4a4.h, no allocation.
 */
#ifndef W4A4_PROBE_H
#define W4A4_PROBE_H

#include <stdint.h>

#include "w4a4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core probe kinds */
enum {
  W4A4_PROBE_INT8 = 0,   /* v_mfma_i32_32x32x32_i8 */
  W4A4_PROBE_FP8 = 1,    /* v_mfma_scale_f32_32x32x64_f8f6f4, FP8 E4M3 operands */
  W4A4_PROBE_FP6 = 2,    /* the same, FP6 E2M3 operands (the INT4 GEMM's instruction) */
  W4A4_PROBE_FP4 = 3,    /* the same, FP4 E2M1 operands (the MXFP4 GEMM's instruction) */
  W4A4_PROBE_FP16 = 4,   /* v_mfma_f32_32x32x16_f16 (the NVFP4 GEMM's instruction) */
  W4A4_PROBE_VALU_F32 = 5 /* v_fma_f32 on the vector unit (the INT4 GEMM's group epilogue) */
};

/* Bytes of device memory the `sink` of either probe must hold (host-only). */
int64_t w4a4_probe_sink_bytes(void);

/* Useful operations (2 per multiply-add) one w4a4_probe_mfma launch of
 * `iters` iterations performs, or -1 for an unknown kind (host-only). */
int64_t w4a4_probe_mfma_ops(int32_t kind, int64_t iters);

/*
 * A grid of waves issuing `iters` x 4 independent MFMAs of `kind` each on
 * pseudo-random operand bits (the matrix cores' clock depends on the data),
 * or, for W4A4_PROBE_VALU_F32, 64 independent fp32 fmas per lane per
 * iteration (w4a4_probe_mfma_ops counts 2 ops per fma).
 *   iters  > 0;  sink  out: w4a4_probe_sink_bytes() bytes, 4-byte aligned
 */
w4a4_status_t w4a4_probe_mfma(int32_t kind, int64_t iters, void* sink, void* stream);

/*
 * Stream `bytes` of buf through the vector memory path (16-byte loads,
 * grid-stride, XOR-folded into sink).  bytes > 0, bytes % 16 == 0;
 * buf 16-byte aligned; sink as above.
 */
w4a4_status_t w4a4_probe_hbm_read(const void* buf, int64_t bytes, void* sink, void* stream);

/* Copy `bytes` from src to dst (16-byte loads and stores, grid-stride). */
w4a4_status_t w4a4_probe_hbm_copy(const void* src, int64_t bytes, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_PROBE_H */
