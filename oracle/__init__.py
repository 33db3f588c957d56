"""CPU oracle for the gated delta rule -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
anything from this package.  It shares no code with the GPU library.
"""
