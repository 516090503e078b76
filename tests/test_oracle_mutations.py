"""The oracle's pins catch planted mistakes (CPU only).

Each case runs pin tests of the oracle (their own test files, unchanged: those of the decoders,
act_quant and the GEMM reference for the core functions; those of the bf16 rounding, the
quantized outputs, the MXFP4 producer, the epilogues and the backward-pass operands for theirs)
in a child pytest process with one mistake planted in the oracle by the
`oracle_mutants` plugin (tests/oracle_mutants.py names each one), and requires that at least one
pin fails.  A control run with nothing planted must pass, so a failure under a mutant is the
mutant's doing.  This shows the pins tie the oracle to the pages and to the mathematics, not
only to itself: a dropped bias, a transposed operand or block-scale index, a wrong nibble order,
exponent bias, subnormal step, scale ceiling, floor or tie rule, a lost sign of zero, a table
typo, a loosened acceptance bound; in the later functions a truncating or ties-away bf16
rounding, a swapped nibble pack, the wrong E2M1 maximum, an erfc argument's sign, a dropped
residual, a Philox round or multiplier bit, the word order of the random stream, a <= for < in
stochastic rounding, a missing transpose, and each acceptance bound's terms.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = {"core": ["tests/test_oracle_decoders.py", "tests/test_oracle_act_quant.py",
                 "tests/test_oracle_gemm.py"],
        "next": ["tests/test_oracle_quant_out.py", "tests/test_oracle_act_quant_fp4.py",
                 "tests/test_oracle_epilogue.py", "tests/test_oracle_grad.py",
                 "tests/test_oracle_quant_fp4_out.py"]}


def _run_pins(job) -> subprocess.CompletedProcess:
    mutant, group = job
    env = dict(os.environ, ORACLE_MUTANT=mutant,
               PYTHONPATH=os.pathsep.join([HERE, ROOT, os.environ.get("PYTHONPATH", "")]),
               OMP_NUM_THREADS="2", OPENBLAS_NUM_THREADS="2", MKL_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "oracle_mutants",
                           "-p", "no:cacheprovider", "-m", "not gpu", *PINS[group]],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.fixture(scope="module")
def results():
    jobs = [("none", "core"), ("none", "next")] + [(n, g) for n, (_, g) in MUTANTS.items()]
    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(zip(jobs, ex.map(_run_pins, jobs)))


def _failed(r: subprocess.CompletedProcess):
    return [line.split(" ")[1] for line in r.stdout.splitlines() if line.startswith("FAILED ")]


@pytest.mark.parametrize("group", sorted(PINS))
def test_control_run_passes(results, group):
    r = results[("none", group)]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(results, mutant):
    r = results[(mutant, MUTANTS[mutant][1])]
    assert r.returncode == 1, (f"{mutant}: the pins did not fail (exit {r.returncode})\n"
                               + r.stdout[-2000:] + r.stderr[-2000:])
    assert _failed(r), r.stdout[-2000:]
