"""CPU oracle for the Llama-3 decoder forward pass.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product package.

``oracle.llama`` is the fp64 numpy oracle; ``oracle.brute`` is a scalar
pure-Python second formulation used to check it on tiny shapes.
``oracle.runner`` binds the oracle to the seeded inputs of ``inputs``.

Parity status: every function is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py``.  The end-to-end stack is pinned only through
its parts and the invariants those tests check (the pages' only worked
example needs trained weights that are not available).
"""
from . import llama, brute  # noqa: F401
