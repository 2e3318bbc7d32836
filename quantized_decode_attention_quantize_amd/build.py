"""Build libkvq.so (HIP, gfx950) in-tree.

Every translation unit is compiled for gfx950 only, with packed-FP32
instruction selection disabled, IEEE-correct fp32 division and square root,
and denormals kept.  The quantiser translation unit is also compiled without
floating-point contraction: its codes must be bit-identical to the format's
fp32 definition.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkvq.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]
# The decode kernels keep their MFMA accumulators in ordinary VGPRs (the
# VGPR form of the MFMA instructions): the folded scores are read by VALU
# right after each MFMA, and with the accumulators in AGPRs every read was an
# extra v_accvgpr_read (8 per page pair, 64 more per rescale).  Measured:
# 0.35 us less per 16K split-kernel launch, 208 -> 172 registers.
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCES = {
    "kvq_append.hip": ["-ffp-contract=off"],
    "kvq_balance.hip": ["-ffp-contract=off"],
    "kvq_decode.hip": MFMA_VGPR,
    "kvq_fp16.hip": MFMA_VGPR,
    "kvq_api.hip": [],
    "kvq_probe.hip": [],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkvq")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
