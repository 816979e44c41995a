"""This GPU's own peaks, from the library's probe kernels (include/w4a4_probe.h):
back-to-back MFMAs of each kind on pseudo-random operands, fp32 vector fmas,
and HBM read / copy streams. Measurement only (roofline fractions against the
measured peaks beside the data-sheet ones; the granularity policy's rho)."""
from __future__ import annotations

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 matrix-core peak (5.0 POP/s)
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4/fp6 matrix-core peak
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 matrix-core peak
PEAK_HBM_GBS = 8000.0

PROBE_KINDS = {"int8": 0, "fp8": 1, "fp6": 2, "fp4": 3, "fp16": 4, "valu_f32": 5}
# data-sheet figures; the vector unit's fp32 figure is reached by scalar
# (non-packed) v_fma_f32 issued from several waves per SIMD (measured: one
# wave alone issues an fma every ~4 cycles, several every ~2)
VENDOR_PEAKS = {"int8_tops": PEAK_INT8_TOPS, "fp8_tflops": 5000.0, "fp6_tflops": PEAK_FP4_TFLOPS,
                "fp4_tflops": PEAK_FP4_TFLOPS, "fp16_tflops": PEAK_FP16_TFLOPS, "valu_f32_tflops": 157.3,
                "hbm_gbs": PEAK_HBM_GBS}


def measure_peaks(iters: int = 16000, reps: int = 3, hbm_bytes: int = 2 << 30):
    """This GPU's own peaks, from the library's probe kernels (w4a4_probe.h):
    back-to-back MFMAs of each kind on pseudo-random operands, independent
    fp32 vector fmas, and HBM read / copy streams over buffers 8x the 256 MB
    last-level cache. Best of ``reps`` HIP-event-timed launches after one
    warm-up; units TOPS / TFLOP/s / GB/s."""
    import torch
    from . import _lib
    lib = _lib.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.empty(lib.w4a4_probe_sink_bytes() // 4, dtype=torch.float32, device="cuda:0")
    out = {}

    def best_seconds(launch):
        launch()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            dt = e0.elapsed_time(e1) / 1e3
            best = dt if best is None else min(best, dt)
        return best

    for name, kind in PROBE_KINDS.items():
        sec = best_seconds(lambda: _lib.call("w4a4_probe_mfma", kind, iters, sink.data_ptr(), stream))
        unit = "tops" if name == "int8" else "tflops"
        out[f"{name}_{unit}"] = lib.w4a4_probe_mfma_ops(kind, iters) / sec / 1e12
    buf = torch.empty(hbm_bytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    sec = best_seconds(lambda: _lib.call("w4a4_probe_hbm_read", buf.data_ptr(), hbm_bytes, sink.data_ptr(), stream))
    out["hbm_read_gbs"] = hbm_bytes / sec / 1e9
    half = hbm_bytes // 2
    dst = torch.empty(half // 4, dtype=torch.float32, device="cuda:0")
    sec = best_seconds(lambda: _lib.call("w4a4_probe_hbm_copy", buf.data_ptr(), half, dst.data_ptr(), stream))
    out["hbm_copy_gbs"] = 2 * half / sec / 1e9
    del buf, dst
    torch.cuda.synchronize()
    return out
