"""CPU oracle for the whole-step programs -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library does not depend on it.
"""
