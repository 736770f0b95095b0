"""The oracle's pins catch plausible mistakes in it.

Each entry of ``tests/oracle_mutants.py`` plants one slip in one oracle
function (a dropped scale term, a strict instead of an inclusive causal
test, a swapped block index, an interleaved GQA head mapping, a natural
instead of a base-2 exponent, the listing's inclusive cumulative sum, ...).
A child pytest run of the pins of that function, with the slip in place,
must fail.  Runs on the CPU only; the oracle is changed in the child
processes alone.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

from tests import oracle_mutants

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(name):
    files, _ = oracle_mutants.MUTANTS[name]
    env = dict(os.environ, BSATTN_ORACLE_MUTANT=name, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", *[os.path.join("tests", f) for f in files],
           "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, (r.stdout + r.stderr)[-600:]


def test_every_planted_mistake_fails_a_pin():
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run, sorted(oracle_mutants.MUTANTS)))
    # pytest exits 1 when a test failed; 0 would mean the slip went unnoticed,
    # anything else that the child run itself broke
    survived = [(n, out) for n, rc, out in results if rc == 0]
    broken = [(n, rc, out) for n, rc, out in results if rc not in (0, 1)]
    assert not survived, "mistakes no pin catches: " + ", ".join(n for n, _ in survived)
    assert not broken, broken
