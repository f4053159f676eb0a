"""TEST INFRASTRUCTURE ONLY: the CPU oracle (plain C + a ctypes front).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP product path never imports or links it.
"""
