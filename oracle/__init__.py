"""CPU oracle for forward convolution (fp64, direct nested loops).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library never does.
Parity status of every function is stated in ref.py and check.py.
"""
