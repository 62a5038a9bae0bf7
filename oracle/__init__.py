"""Test oracle for the BaKron solve -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU statement of what the
BaKron solver computes, in float64.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import,
call, link or run anything under ``oracle/``.  The HIP library never does,
and shares no code, header, table or helper with it.

Pages cited (by title):

* [S]  paper summary "FastKron: Efficient Quantization with Kronecker-Factored
       Hessians" (arXiv 2608.06291): setup paragraph, the derivation
       naive -> antidiagonal -> BaKron, Proposition 3.1, Theorem 3.2,
       Corollary 3.4, Table 3.
* [A]  paper page "BaKron: Efficient Quantization with Kronecker-Factored
       Hessians": abstract.
* [N5] news article "BaKron Reduces Two-Sided Hessian Quantization to Cubic
       Complexity, With Its 8192-Square-Matrix Kernel 60x Faster Than
       YAQA": GPTQ as the A (x) I special case, benchmark setup.

Modules:

* ``reference`` -- numpy float64 forms: brute-force GPTQ on vec(W) with the
  explicit Kronecker Hessian, BaKron-naive (any order), BaKron-antidiagonal,
  the inverse-free "L-form", the factor step, the objective, and a validator
  that checks any claimed output against the method at any size.
* ``recursive`` -- ctypes front end of ``recursive.c``, a C float64
  sequential BaKron-recursive (quadtree divide and conquer) for large shapes.

Parity status: every function here is pinned by tests in ``tests/``
(``test_oracle_*.py``) against brute force, closed forms, hand-worked
fixtures in ``tests/golden/`` or special cases; none is "parity unpinned".
"""
