"""fp64 CPU oracle for WildCat coreset attention (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package; the HIP product path never does.
"""
