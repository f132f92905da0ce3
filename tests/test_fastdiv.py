"""The quantizer's two division shortcuts are exact: an exhaustive CPU check
(C with hardware fma) over every input they can receive."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_division_shortcuts_exhaustive(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.check_call(["gcc", "-O3", "-march=native", "-fopenmp", "-ffp-contract=off",
                           os.path.join(HERE, "fastdiv_check.c"), "-o", str(exe), "-lm"])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "divide by 255: 0 mismatches" in r.stdout
    assert "reciprocal: 0 mismatches" in r.stdout
