"""fp64 CPU oracle of the routed MoE FFN layer (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library.
"""
from .moe import *  # noqa: F401,F403
from .moe import __all__  # noqa: F401
