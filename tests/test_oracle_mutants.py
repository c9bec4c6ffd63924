"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is the oracle source compiled with -DORACLE_MUTANT=n, which
changes one line into a plausible slip (dropped term, wrong sign, wrong
exponent, wrong index, wrong factor).  The pin suite is then run against the
mutant in a child process and must fail.  Everything here runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    1: "drops the cross-electron term of the recurrence",
    2: "flips the sign of the (W-P)/(W-Q) term",
    3: "uses rho/eta instead of rho/zeta on the bra side",
    4: "uses 2m+3 instead of 2m+1 in the Boys downward recursion",
    5: "drops the v-dependent sign of the spherical coefficients",
    6: "uses (4 alpha)^((l+1)/2) instead of (4 alpha)^(l/2) in the primitive normalisation",
    7: "uses P-A instead of P-B when raising b",
    8: "forgets the factor 2 for off-diagonal density pairs in J",
    9: "drops the factor 2 of 2 alpha in the centre derivative",
}


@pytest.mark.parametrize("mut", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mut, tmp_path):
    so = str(tmp_path / f"liberi_oracle_mut{mut}.so")
    oracle.build(out=so, defines=[f"ORACLE_MUTANT={mut}"])
    env = dict(os.environ, ERI_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {mut} ({MUTANTS[mut]}) passed every pin:\n{r.stdout[-2000:]}"
