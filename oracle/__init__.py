"""fp64 CPU oracle for PISA piecewise sparse attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the HIP library never does.
"""
from .pisa_oracle import *  # noqa: F401,F403
from .pisa_oracle import __all__  # noqa: F401
