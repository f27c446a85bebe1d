"""fp64 CPU oracle for the mHC hot path — test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg may use it;
the HIP library never imports or calls it.
"""
from . import mhc_oracle  # noqa: F401
