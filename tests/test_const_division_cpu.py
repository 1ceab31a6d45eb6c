"""The shortcut division by 6 and 12 of the WENO kernels (CPU only).

The kernels divide by the constants 6 and 12 as a product with the rounded
reciprocal corrected by one fused multiply-add remainder step, and take that
path only where a range check on the tap values shows every dividend to be zero
or at least 2^-124 in magnitude and finite.  const_division_check.c compares
the shortcut with the IEEE quotient over every fp32 dividend of the exponent
fields that can differ (and, by exact scaling, all others); this test runs it
and requires agreement from 2^-124 up, and +0 for -0 (the IEEE quotient is -0;
the kernels never pass the sign of a zero candidate on).
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_shortcut_equals_ieee_division(tmp_path):
    exe = str(tmp_path / "const_division_check")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", os.path.join(HERE, "const_division_check.c"),
           "-o", exe, "-lm"]
    if "fma" in open("/proc/cpuinfo").read().split():
        cmd.insert(2, "-mfma")  # hardware fma; libm's fmaf is exact either way
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    fields = [int(f) for f in re.findall(r"from exponent field (\d+)", r.stdout)]
    assert len(fields) == 2 and max(fields) <= 3, r.stdout
    # the shortcut does miss for some subnormal quotients: the check would see a broken comparison
    assert all(int(n) > 0 for n in re.findall(r": (\d+) x disagree", r.stdout)), r.stdout
    # -0 comes out +0 (documented; the kernels never pass a zero's sign on)
    assert r.stdout.count("-0 gives +0 (IEEE -0)") == 2, r.stdout
