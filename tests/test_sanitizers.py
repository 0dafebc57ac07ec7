"""AddressSanitizer and UBSan over the host code (CPU only, no GPU):

* the oracle (both accumulation builds) and the input generator, built with
  gcc -fsanitize=address,undefined, run on small workloads reaching every
  entry point;
* the C ABI library built by hipcc with the sanitizers on its host pass only,
  driven through every argument check and size query of the host ABI tests.

Each run is a child process with the matching sanitizer runtime preloaded
(the interpreter itself is not instrumented); any report fails the test."""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(HERE, "native", "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _gcc_runtime(name):
    return subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()


def test_oracle_and_generator_under_asan_ubsan():
    os.makedirs(BUILD, exist_ok=True)
    for src, out, defs in (("oracle/oracle.c", "liboracle_san.so", []),
                           ("oracle/oracle.c", "liboracle_f64_san.so", ["-DORC_ACC_FP64"]),
                           ("synth/synth.c", "libsynth_san.so", [])):
        subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-ffp-contract=off", *SAN, *defs, os.path.join(ROOT, src),
                               "-o", os.path.join(BUILD, out), "-lm"])
    env = dict(os.environ,
               LD_PRELOAD=f"{_gcc_runtime('libasan.so')}:{_gcc_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, os.path.join(HERE, "native", "sanitized_oracle_run.py"), ROOT, BUILD],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "sanitized oracle run ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_abi_host_checks_under_asan_ubsan():
    rt = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    os.makedirs(BUILD, exist_ok=True)
    so = os.path.join(BUILD, "libmoe_fp4_hostsan.so")
    csrc = sorted(glob.glob(os.path.join(ROOT, "fp4_routed_expert_amd", "csrc", "*.hip")))
    host_san = []
    for f in SAN[:2]:
        host_san += ["-Xarch_host", f]
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-gpu-flush-denormals-to-zero",
           *host_san, "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan",
           "-I", os.path.join(ROOT, "include"), *csrc, "-o", so]
    subprocess.check_call(cmd, stderr=subprocess.DEVNULL)
    env = dict(os.environ, LD_PRELOAD=rt[0], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "native", "sanitized_abi_run.py"), ROOT, so],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "sanitized ABI run ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
