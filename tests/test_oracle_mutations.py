"""The pins catch planted mistakes: the pin suite (tests/test_oracle_pins.py) is run once
per mutant of tests/_mutants.py, each in a child process with the oracle changed in memory,
and every run must fail.  CPU only; the HIP library is not involved."""
import concurrent.futures as cf
import os
import subprocess
import sys

from tests import _mutants

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(name):
    env = dict(os.environ, CSA2_ORACLE_MUTANT=name, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_unmutated_pins_pass():
    name, rc, tail = _run("")
    assert rc == 0, tail


def test_every_planted_mistake_fails_a_pin():
    names = sorted(_mutants.MUTANTS)
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 2)) as ex:
        results = list(ex.map(_run, names))
    survived = [(n, tail) for n, rc, tail in results if rc != 1]  # 1 = some test failed
    assert not survived, "mutants not caught (or the run errored):\n" + "\n".join(f"{n}: {t}" for n, t in survived)
