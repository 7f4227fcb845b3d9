"""Plain CPU oracle for the FP8 scaled linear layer (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP product path never does.
"""
