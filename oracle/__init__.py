"""fp64 CPU oracle for the selective scan (S6) — test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product. The two share no code; the only common module is the
seeded input generator, which holds none of the method's arithmetic.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (values printed on the pages, closed forms,
special cases that reduce to textbook computations, brute force on tiny
inputs) and by the mutation test in ``tests/test_oracle_mutants.py``.
"""
from .oracle import Oracle, build_oracle, default_oracle, ORACLE_SRC  # noqa: F401
