"""Build libgdpa.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python generalized_attention_amd/build.py   (runs without importing the package)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgdpa.so")
PROBE_LIB = os.path.join(HERE, "libgdpa_probe.so")
OBJDIR = os.path.join(HERE, "_build")
BWD_UNITS = [f"gdpa_bwd_{t}_{d}.hip" for t in ("bf16", "f16") for d in (64, 96, 128, 192)]
FUSED_UNITS = [f"gdpa_bwdf_{t}_{d}.hip" for t in ("bf16", "f16") for d in (64, 96, 128)]
SOURCES = FUSED_UNITS + BWD_UNITS + ["gdpa_fwd.hip", "gdpa_fwd_f16.hip", "gdpa_bwd.hip", "gdpa_sched.hip",
                                     "gdpa_api.cpp"]
# Per-source code generation options.  The forward kernels keep their MFMA
# accumulators in architectural VGPRs (the activation reads the S tile with
# no accumulator-to-VGPR copies; the register file still fits two workgroups
# per CU).
# The forward unit streams (up to 40 units at head dims (192, 128)) must unroll
# completely: a partly unrolled stream indexes its register arrays at run time
# and the compiler moves them to scratch or LDS.
EXTRA = {"gdpa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-pragma-unroll-threshold=1000000"],
         "gdpa_fwd_f16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-pragma-unroll-threshold=1000000"]}
# (hipcc's pass that rewrites MFMA register forms fails on the (192, 128)
# backward streams when MFMA results are forced into architectural VGPRs, so
# those units keep the compiler's choice, like the fused units)
EXTRA.update({u: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for u in BWD_UNITS if not u.endswith("_192.hip")})
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libgdpa.so)")


def _flags():
    # Packed fp32 VALU ops are disabled: the kernels use plain fp32 math only.
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wshadow", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + _flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libgdpa.so; always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # throughput probes for bench.py's measured peaks (not part of the GDPA ABI)
    cmd = [_hipcc()] + _flags() + ["-shared", "-o", PROBE_LIB + ".tmp", os.path.join(HERE, "probe", "gdpa_peak.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
