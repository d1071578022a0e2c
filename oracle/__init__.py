"""Independent fp64 CPU oracle of the ETA decode step (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
