"""The oracle's pins catch planted mistakes (CPU only).

Each case runs the pin tests of the decoders, act_quant and the GEMM reference (their own test
files, unchanged) in a child pytest process with one mistake planted in the oracle by the
`oracle_mutants` plugin (tests/oracle_mutants.py names each one), and requires that at least one
pin fails.  A control run with nothing planted must pass, so a failure under a mutant is the
mutant's doing.  This shows the pins tie the oracle to the pages and to the mathematics, not
only to itself: a dropped bias, a transposed operand or block-scale index, a wrong nibble order,
exponent bias, subnormal step, scale ceiling, floor or tie rule, a lost sign of zero, a table
typo, a loosened acceptance bound.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = ["tests/test_oracle_decoders.py", "tests/test_oracle_act_quant.py",
        "tests/test_oracle_gemm.py"]


def _run_pins(mutant: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, ORACLE_MUTANT=mutant,
               PYTHONPATH=os.pathsep.join([HERE, ROOT, os.environ.get("PYTHONPATH", "")]),
               OMP_NUM_THREADS="2", OPENBLAS_NUM_THREADS="2", MKL_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "oracle_mutants",
                           "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.fixture(scope="module")
def results():
    names = ["none", *MUTANTS]
    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(zip(names, ex.map(_run_pins, names)))


def _failed(r: subprocess.CompletedProcess):
    return [line.split(" ")[1] for line in r.stdout.splitlines() if line.startswith("FAILED ")]


def test_control_run_passes(results):
    r = results["none"]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(results, mutant):
    r = results[mutant]
    assert r.returncode == 1, (f"{mutant}: the pins did not fail (exit {r.returncode})\n"
                               + r.stdout[-2000:] + r.stderr[-2000:])
    assert _failed(r), r.stdout[-2000:]
