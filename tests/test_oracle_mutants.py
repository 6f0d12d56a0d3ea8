"""Mutation check of the oracle's pins (no GPU).

Each case plants one plausible mistake in the oracle (tests/_oracle_mutants.py:
a dropped scale, a reversed K index, a wrong exponent bias or table entry, a
swapped nibble or layout index, the tanh form of GELU, a sign error in SiLU,
the bias after the activation, shifted block scales, a truncating rounding,
a metric that ignores the elementwise bound, ...) and runs the oracle's pin
tests in a child process: at least one pin must fail. The control case runs
them with no mistake planted and must pass."""
import os
import subprocess
import sys

import pytest

from tests._oracle_mutants import NAMES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
              if f.startswith("test_oracle_") and f.endswith(".py") and f != "test_oracle_mutants.py")


def _run_pins(mutant):
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    env.pop("ORACLE_MUTANT", None)
    if mutant:
        env["ORACLE_MUTANT"] = mutant
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-p", "tests._oracle_mutants",
           "-m", "not gpu", *PINS]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_pins_pass_without_a_mutant():
    r = _run_pins(None)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("mutant", NAMES)
def test_pins_catch_mutant(mutant):
    r = _run_pins(mutant)
    assert r.returncode == 1 and "failed" in r.stdout, \
        f"no pin failed with mutant {mutant} (rc {r.returncode}):\n{r.stdout[-1500:]}\n{r.stderr[-1500:]}"
