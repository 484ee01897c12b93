"""fp64 CPU oracle for the MTLA hot path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP product path never imports it and shares no code with
it.
"""
from . import mtla  # noqa: F401
from .mtla import *  # noqa: F401,F403
