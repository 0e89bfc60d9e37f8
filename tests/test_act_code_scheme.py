"""The vector product's in-launch activation quantisation decides each E2M1
code from Markstein's corrected quotient |x| / s and the hardware's rounding,
instead of comparing |x| with every midpoint times s.  This CPU check runs
that arithmetic (C, no contraction) against the exact comparisons for every
positive bf16 value and every positive E4M3 scale a block can hold (ratios
up to 2^16, saturated scales included): exhaustive, under a second."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_corrected_quotient_gives_the_exact_code(tmp_path):
    exe = str(tmp_path / "act_code_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "csrc", "act_code_check.c"), "-lm"], check=True)
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(p.stdout)
    assert p.returncode == 0, p.stdout
    bad, total = int(p.stdout.split("bad ")[1].split()[0]), int(p.stdout.split(" of ")[1])
    assert bad == 0 and total > 2_000_000
