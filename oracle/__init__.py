"""CPU fp64 oracle of the VDN attention forward -- test infrastructure only.

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
