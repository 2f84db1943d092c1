"""CPU oracle for the W4A4 rotate / quantize / GEMM path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.  It shares no
code with the HIP library; the two meet only through the seeded inputs in
`workloads`.
"""
from .w4a4 import *  # noqa: F401,F403
from .w4a4 import apply_signs, hadamard, rotate, rotate_normalized  # noqa: F401
