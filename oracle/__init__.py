"""Plain fp64 CPU reference for exact attention -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library and never imports
it; the two meet only through the seeded input generators, which hold none of
the method's arithmetic.
"""
from .oracle import (  # noqa: F401
    attention_forward,
    attention_forward_rows,
    attention_backward,
    build,
    num_threads,
    widen,
)
