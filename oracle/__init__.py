"""CPU oracle for diagonal-batched RMT inference (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the HIP library and its Python binding never do.
"""
