"""Host check of the reciprocal-based FP8 QDQ quotient the GPU kernels use.

The kernels (fake-quant and the combine's fused QDQ) form x / s from the
correctly rounded reciprocal plus one fused-multiply-add correction instead of
dividing.  ``host/qdq_quotient_check.c`` restates that arithmetic in C (gcc
on the host, IEEE binary32 with fmaf) and checks it against the IEEE
quotient for every finite bfloat16 x over a few thousand scales: equal
quotients where they can matter, equal E4M3 codes (sign of zero included)
everywhere.  The GPU parity tests check the kernels themselves against the
oracle; this pins the identity they rely on for scales those tests do not
reach.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc on the host")
def test_reciprocal_quotient_matches_ieee_division(tmp_path):
    exe = tmp_path / "qdq_quotient_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "host", "qdq_quotient_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe), "11", "300"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    checked = int(r.stdout.split("checked")[1].split()[0])
    assert checked > 100_000_000, r.stdout
