"""Every planted oracle mistake (tests/oracle_mutations.py) must make the pin suite fail.
Each mutation runs the pins in a fresh interpreter so that no mutation leaks; the
interpreters run side by side (one per CPU, at most 8) and each case checks its own."""
import concurrent.futures
import os
import subprocess
import sys

import pytest

from tests.oracle_mutations import MUTATIONS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_pins.py", "tests/test_pool_replay.py", "tests/test_oracle_properties.py"]


def _run(name):
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from tests import oracle_mutations as M\n"
        "M.apply(%r)\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + %r))\n"
    ) % (ROOT, name, PINS)
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                          timeout=600, env=env)


@pytest.fixture(scope="module")
def outcomes():
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        return dict(zip(sorted(MUTATIONS), ex.map(_run, sorted(MUTATIONS))))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, outcomes):
    r = outcomes[name]
    assert r.returncode == 1, (name, r.returncode, r.stdout[-2000:], r.stderr[-2000:])
