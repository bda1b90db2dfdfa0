"""CPU fp64 oracle for JoLT / FlashJoLT KV-cache compression.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The product path (the HIP library and its Python binding) never touches
it and shares no code with it.

It follows Krishnan & Schulz, "A JoLT for the KV Cache: Near-Lossless KV Cache
Compression via Joint Rank-bit Allocation" (arXiv 2607.12550v2), Sec. 3 and
Sec. 3.1, step by step in numpy float64 with LAPACK routines as primitives.

Parity pins: every public function is pinned by ``tests/test_oracle_*.py``
against facts the pages or the mathematics fix (printed eps^2 calibration,
4.25 bits/element, Eckart-Young / ST-HOSVD identities, brute-force allocation,
published SplitMix64 outputs).  Nothing here is "parity unpinned".
"""
from . import rng  # noqa: F401
from .jolt import *  # noqa: F401,F403
from . import decode  # noqa: F401,E402
