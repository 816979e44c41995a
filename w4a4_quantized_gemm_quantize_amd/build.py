"""Build libw4a4.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m w4a4_quantized_gemm_quantize_amd.build

Compiles every ``csrc/*.hip`` with hipcc into ``_build/`` and links the shared
library next to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a4.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-Rpass-analysis=kernel-resource-usage",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

# The debug entry points' kernels (partials export) may spill; production
# kernels must not: a spill there costs a multiple of the kernel time (the
# per-token GEMM variant once ran 4x slower on 87 spilled registers).
def _is_debug_kernel(name: str) -> bool:
    """A partials-export instantiation: PARTIALS is the first template argument
    of the INT4 and NVFP4 kernels and the last one of the MXFP4 kernel."""
    return ("11k_w4a4_gemmILb1E" in name or "17k_w4a4_gemm_smallILb1E" in name
            or "12k_nvfp4_gemmILb1E" in name
            or ("12k_mxfp4_gemm" in name and name.endswith("Lb1EEEvNS0_6ParamsE")))


def _scratch_report(out: str):
    """(kernel, scratch bytes per lane) pairs from the resource-usage remarks."""
    res, name = [], None
    for ln in out.splitlines():
        if "remark: Function Name:" in ln:
            name = ln.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in ln and name:
            res.append((name, int(ln.split("ScratchSize [bytes/lane]:")[1].split()[0])))
            name = None
    return res


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in sources]

    def compile_one(pair):
        src, obj = pair
        return _run([hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj])

    spills = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        for out in ex.map(compile_one, zip(sources, objs)):
            for name, scratch in _scratch_report(out):
                if scratch and not _is_debug_kernel(name):
                    spills.append((name, scratch))
            warn = "\n".join(ln for ln in out.splitlines() if "remark:" not in ln)
            if verbose and warn.strip():
                print(warn)
    if spills:
        raise RuntimeError("production kernels use scratch (register spills): "
                           + ", ".join(f"{n} ({b} B/lane)" for n, b in spills))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
