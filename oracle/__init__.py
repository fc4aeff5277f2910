"""Plain CPU oracle for the DSA forward path.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package; the product path may
not, and shares no code with it.
"""
