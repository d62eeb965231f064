"""The MSA oracle: plain fp64 CPU implementation used to check the HIP path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP library (``routed_sparse_attention_amd``) and neither imports the
other.

Pinning status (what checks the oracle against something other than itself is
listed in ``tests/test_oracle_pins.py``): every public function is pinned by a
closed form, an invariant, brute force, or an independent library routine.
"""
from .msa_oracle import *  # noqa: F401,F403
from . import msa_oracle  # noqa: F401
