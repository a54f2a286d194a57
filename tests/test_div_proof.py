"""Exhaustive CPU proof that the kernels' reciprocal-based division equals IEEE binary32
division x / s for every bf16 mantissa of x and every binary32 mantissa of s (and the
per-group scale for every bf16 amax).  Builds tests/cpu/div_proof.cpp against the
library's own fp8q_math.h with the host compiler."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.slow
def test_reciprocal_division_is_correctly_rounded(tmp_path):
    exe = tmp_path / "div_proof"
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fopenmp",
                    "-I", os.path.join(ROOT, "fp8_e4m3_quantization_amd", "csrc"),
                    os.path.join(HERE, "cpu", "div_proof.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    for line in r.stdout.splitlines():
        assert line.endswith(" 0"), line
