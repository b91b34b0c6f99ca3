"""CPU oracle for the LongCat Sparse Attention (LSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.

``lsa_oracle`` is the float64 numpy oracle (one function per step of the method).
``loops`` is a pure-Python brute-force restatement for tiny inputs, used to
cross-check the numpy oracle.
"""
