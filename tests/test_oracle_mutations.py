"""Every planted oracle mistake (tests/oracle_mutations.py) must make the pin suite fail.
Each mutation runs the pins in a fresh interpreter so that no mutation leaks."""
import os
import subprocess
import sys

import pytest

from tests.oracle_mutations import MUTATIONS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_pins.py", "tests/test_pool_replay.py"]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from tests import oracle_mutations as M\n"
        "M.apply(%r)\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + %r))\n"
    ) % (ROOT, name, PINS)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, (name, r.returncode, r.stdout[-2000:], r.stderr[-2000:])
