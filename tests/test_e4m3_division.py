"""The e4m3 encoders divide by the scale with a short exact sequence instead
of an IEEE division; this checks, exhaustively on the host, that it yields
the code of the correctly rounded quotient for every bf16 value and every
scale a bf16 maximum can give (the C program states the sequence)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "e4m3_division_check.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_e4m3_division_matches_correctly_rounded_quotient(tmp_path):
    exe = str(tmp_path / "e4m3_division_check")
    # no contraction: every product and fma in the program is the one it names
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
    nparts = max(1, min(8, os.cpu_count() or 1))
    procs = [subprocess.Popen([exe, str(p), str(nparts)], stdout=subprocess.PIPE, text=True) for p in range(nparts)]
    pairs = bad = 0
    for p in procs:
        out, _ = p.communicate(timeout=600)
        last = out.strip().splitlines()[-1].split()
        pairs += int(last[0])
        bad += int(last[1])
        assert p.returncode == 0, out
    # every pair (a, x) with |x| <= a over the 32640 positive finite bf16 maxima
    assert pairs > 1_000_000_000
    assert bad == 0
