"""CPU proof for the kernels' q-quantisation division (no GPU needed).

The fp8 path divides each bf16 q element by the tile scale with a three-op
FMA-corrected product instead of an IEEE division.  tests/native/
check_div_by_scale.c replays that exact sequence for every bf16 tile maximum
and every bf16 element of the tile (about 1e9 pairs) and checks that the OCP
e4m3 code is the one the IEEE quotient gives -- the quotient the oracle uses.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_fast_division_gives_ieee_e4m3_codes(tmp_path):
    exe = tmp_path / "check_div_by_scale"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-mfma", "-o", str(exe),
                    os.path.join(HERE, "native", "check_div_by_scale.c"), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 give different e4m3 codes" in r.stdout
