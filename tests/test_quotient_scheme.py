"""The weight quantiser's fast path divides by a per-block value with three
fp32 operations (a product, an exact fused residual, a fused correction)
instead of a division.  This CPU check runs that arithmetic (C, no
contraction) against correctly rounded division on a strided sweep of every
case the code decisions depend on; the same program with stride 1 is the
exhaustive run (minutes)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_corrected_quotient_matches_division(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "csrc", "quotient_check.c"), "-lm"], check=True)
    p = subprocess.run([exe, "509", "-99", "-40", "-10", "0", "20", "100"], capture_output=True,
                       text=True, timeout=300)
    print(p.stdout)
    assert p.returncode == 0, p.stdout
    lines = p.stdout.strip().splitlines()
    assert len(lines) == 13
    for line in lines:
        bad, total = int(line.split("bad ")[1].split()[0]), int(line.split(" of ")[1])
        assert bad == 0 and total > 10000, line
