"""fp64 CPU oracles of the routed MoE FFN layer and of the 4-bit KV-cache
codec with sparse attention (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library.
"""
from .kv import *  # noqa: F401,F403
from .kv import __all__ as _kv_all
from .moe import *  # noqa: F401,F403
from .moe import __all__ as _moe_all

__all__ = list(_moe_all) + list(_kv_all)
