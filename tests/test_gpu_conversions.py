"""The gfx950 conversion instructions the kernels round with, checked on the
GPU against the library's rounding rules over every input they can receive.

The MXFP8 element rule of the OCP MX v1.0 conversion (e4m3, round to nearest
even, saturating) and bf16 round-to-nearest-even are what the oracle computes;
the kernels use v_cvt_pk_fp8_f32 (after a clamp to +-448) and
v_cvt_pk_bf16_f32 instead of bit manipulation.  tests/native/cvt_equivalence
runs each fp32 input with |x| < 512 (e4m3) and each finite fp32 input (bf16)
through both and counts differences.  The program is built by
__graft_entry__.build() on the CPU.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "native", "_build", "cvt_equivalence")


@pytest.mark.gpu
def test_hardware_conversions_match_rounding_rules():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    seen = {}
    for line in r.stdout.splitlines():
        parts = line.split()
        if len(parts) == 5 and parts[1] == "inputs" and parts[3] == "mismatches":
            seen[parts[0]] = (int(parts[2]), int(parts[4]))
    assert seen.get("e4m3") == (2 * 0x44000000, 0), r.stdout
    assert seen.get("bf16") == (2 * 0x7F7F8000, 0), r.stdout
