"""The oracle's pins are strong enough: each plausible mistake planted in the
oracle (tests/oracle_mutants.py: dropped terms, wrong signs, indices and
exponents, transposed operands, rounding modes) makes at least one of them
fail.  Each mistake runs the pin files in a subprocess of its own (the
mistake is applied at import, through BEAM_ORACLE_MUTANT), and the unmodified
oracle passes the same run."""
import concurrent.futures as cf
import os
import subprocess
import sys

import oracle_mutants

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_select.py", "tests/test_oracle_invariants.py",
             "tests/test_oracle_attention.py", "tests/test_oracle_dense.py", "tests/test_oracle_fp8.py"]


def run_pins(name):
    env = dict(os.environ)
    env.pop("BEAM_ORACLE_MUTANT", None)
    if name:
        env["BEAM_ORACLE_MUTANT"] = name
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return name, r.returncode, (r.stdout + r.stderr)[-1500:]


def test_every_planted_mistake_fails_a_pin():
    names = [None] + sorted(oracle_mutants.MUTANTS)
    with cf.ThreadPoolExecutor(4) as ex:
        results = list(ex.map(run_pins, names))
    control = results[0]
    assert control[1] == 0, f"the unmodified oracle fails its pins:\n{control[2]}"
    survivors = [n for n, rc, _ in results[1:] if rc == 0]
    assert not survivors, f"mistakes no pin catches: {survivors}"
    # a pin must fail (status 1), not the run itself (collection or usage errors)
    broken = [(n, rc, out) for n, rc, out in results[1:] if rc != 1]
    assert not broken, broken[:2]
    assert len(results) - 1 >= 25
