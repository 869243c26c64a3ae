"""The per-row quantizer divides by the row's scale through its correctly rounded reciprocal
and an exact fma remainder (one IEEE division per row); this checks on the CPU that the
result is the correctly rounded quotient over the quantizer's whole input domain, so the
kernel's codes equal rint(x / s). Compiled with gcc, no GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_reciprocal_remainder_quotient(tmp_path):
    exe = str(tmp_path / "quotient_identity")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "quotient_identity.c"), "-lm"], check=True)
    r = subprocess.run([exe, "300"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 mismatches" in r.stdout
