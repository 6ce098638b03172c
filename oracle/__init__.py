"""CPU fp64 oracle for shared-prefix fork / DAG attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library; the two meet only
in the seeded inputs drawn by ``workloads``.

Modules (each function cites the page passage it follows):
  pagetable  -- flat page pool + per-sequence block tables, refcounts, fork,
                mount, copy-on-write, drop / repos, rewind, release
  attention  -- materialising decode attention and the log-sum-exp merge
  rope       -- rotary re-rotation used by Repos
  prefill    -- DAG visibility rule, block counts and dense masked attention

Readings taken where the pages are silent are listed in each module header.
Every function here is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, library routines, brute force and the one worked example the pages
print (Agentrix page sharing); none is marked "parity unpinned".
"""
from . import attention, pagetable, prefill, rope  # noqa: F401
