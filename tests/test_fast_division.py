"""Host check of the quantisers' division shortcut (see tests/fast_div_check.c):
the corrected product x * RN(1/scale) gives the same INT8 and E4M3 codes as the
IEEE quotient x / scale for every scale >= 2^-80.  The GPU tests check the
kernels' codes against the oracle bit for bit; this pins the arithmetic
argument on far more operands than they reach."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_corrected_division_gives_the_ieee_codes(tmp_path):
    exe = str(tmp_path / "fast_div_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "fast_div_check.c"), "-o", exe, "-lm"],
                   check=True)
    r = subprocess.run([exe, "120"], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
