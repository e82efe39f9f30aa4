"""Host check of the division steps the GPU quantiser takes: the scale
m/448 and the quotients v/s from a correctly rounded reciprocal and one FMA
residual step equal the IEEE results wherever the kernel uses them (it
divides elsewhere), up to the sign-correct e4m3 zeros of tiny quotients."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_residual_step_division_is_exact(tmp_path):
    exe = str(tmp_path / "div_step")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "cpu_checks", "div_step.c"), "-lm"], check=True)
    out = subprocess.run([exe, "6000000"], check=True, capture_output=True, text=True).stdout
    checked, bad = map(int, out.split())
    assert checked > 2_000_000
    assert bad == 0
