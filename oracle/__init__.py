"""fp64 CPU oracle for paged low-rank-compressed attention (test infrastructure only).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may import
this package.  It shares no code with the HIP library.
"""
from .starkv_oracle import *  # noqa: F401,F403
