"""The write kernels take the IEEE quotient fl(y / scale) that the int4 /
int8 / fp8 rules round without a division per element (a correctly rounded
reciprocal and two fmas, Markstein's correction). tests/host/quotient_identity.c
checks, for the (absmax, y) pairs the write path can meet, that the codes
equal those of the IEEE quotient; here over every 13th absmax (all y of it,
both signs, all three modes), built with gcc without fast-math or fp
contraction. (Run with stride 1 it covers every pair: 0 mismatches.)"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_division_free_quotient_matches_ieee(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "qid")
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "host", "quotient_identity.c"), "-lm"], check=True)
    r = subprocess.run([exe, "13"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
