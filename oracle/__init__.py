"""CPU oracle for the SkipLayerNormalization row operator (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product path never imports it.
"""
