"""Host check of the division step the GPU quantiser takes: a correctly
rounded reciprocal and one FMA residual step give the IEEE quotient bit for
bit on the domain where the kernel uses them (it divides elsewhere)."""
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
    assert checked > 1_000_000
    assert bad == 0
