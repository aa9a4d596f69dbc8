"""Each planted oracle mistake (tests/oracle_mutants.py) must make the oracle's
pin suite (tests/test_oracle.py) fail.  CPU only: one pytest subprocess per
mutant."""
import os
import subprocess
import sys

import pytest

from tests.oracle_mutants import MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_pins(mutant):
    env = dict(os.environ, CALIBATTN_ORACLE_MUTANT=mutant)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle.py")],
                          cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                          timeout=600)


def test_unmutated_pins_pass():
    r = _run_pins("")
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant):
    r = _run_pins(mutant)
    assert r.returncode != 0, f"mutant {mutant} survived the oracle pins:\n{r.stdout[-1500:]}"
