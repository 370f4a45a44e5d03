"""CPU oracle for HOT/COLD decode attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct reference implementations used to check the
HIP path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here; the
product library never does, and this package imports nothing from it.

Modules
  alloc      COLD block pool (refcounts, free stack, copy-on-write, fork,
             release) and HOT contiguous first-fit slab pool.
  attention  fp64 softmax attention over the logical concatenation of a
             request's prefix and suffix tokens; the log-sum-exp merge.
  pools      numpy mirror of the device KV pools: HOT slab addressing,
             slot addressing, reshape_and_cache, copy_blocks, paged gather.
  costmodel  the pages' byte / FLOP model and the effective-M rule.
  driver     runs a drawn workload through the oracle allocators and pools.

Pinned by tests in ``tests/test_oracle_*.py`` against values and closed forms
fixed by the pages and by mathematics (see each module's header for what pins
it).  Every function here has such a pin.  What stays unpinned is a reading,
not a function: the HOT pool's eviction tie-break beyond least recently
released first (lower base on equal ticks, which cannot occur since ticks are
unique) has no value on the pages to check against.
"""
