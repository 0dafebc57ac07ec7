"""Build libmoe_fp4.so (gfx950) in-tree with hipcc.

Each ``csrc/*.hip`` is compiled to an object in parallel, then linked into
``fp4_routed_expert_amd/libmoe_fp4.so``.  Run ``python -m fp4_routed_expert_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
SO = os.path.join(HERE, "libmoe_fp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep fp32 subnormals (the MXFP8 rule is exact down to bf16 subnormals)
    "-fno-gpu-flush-denormals-to-zero",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = SO + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SO)
    if verbose:
        print("built", SO)
    return SO


# Stand-alone GPU programs under tests/native, built here (on the CPU) so that
# GPU runs only execute them: the conversion check of the test suite and the
# two measurement probes whose rocprofv3 summaries are in profiles/.
CHECKS = {
    os.path.join(ROOT, "tests", "native", name + ".hip"): os.path.join(ROOT, "tests", "native", "_build", name)
    for name in ("cvt_equivalence", "hbm_stream", "mfma_rate", "lds_port")
}


def build_checks(verbose: bool = False) -> None:
    for src, exe in CHECKS.items():
        os.makedirs(os.path.dirname(exe), exist_ok=True)
        flags = [f for f in HIP_FLAGS if f not in ("-fPIC",)]
        cmd = [HIPCC, *flags, "-I", CSRC, src, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print("built", exe)


if __name__ == "__main__":
    build(verbose=True)
    build_checks(verbose=True)
    sys.exit(0)
