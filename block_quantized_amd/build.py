"""Build libqmm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every translation unit is compiled by hipcc for gfx950 only, with packed-fp32
instruction selection disabled.  The codec unit (quantize/dequantize) is
built with -ffp-contract=off because its results are defined to the bit;
the product kernels keep the default contraction.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqmm.so")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
UNITS = {
    "codec.hip": ["-ffp-contract=off"],
    "gemv.hip": [],
    # MFMA results in VGPRs (not AGPRs): the epilogue reads them without
    # v_accvgpr_read, and register use drops enough for 2 waves per SIMD
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "probe.hip": [],
    "qmm.cpp": [],
}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every unit and link libqmm.so (always recompiles)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    units = {u: f for u, f in UNITS.items() if os.path.exists(os.path.join(CSRC, u))}
    with cf.ThreadPoolExecutor(max_workers=min(8, len(units))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), units.items()))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host stub failed to emit must fail the
    # build here, not the first dlopen
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
