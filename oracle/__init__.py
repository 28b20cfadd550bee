"""CPU oracle for the GrowPage capacity-boundary engine.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``demand_paged_kv_amd``) never imports, links or runs it, and the two share no
code: the oracle is a plain, slow, float64 numpy restatement of what the pages
describe, used to check the HIP kernels element by element.
"""
from .growpage_oracle import *  # noqa: F401,F403
