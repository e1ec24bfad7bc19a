"""fp64 CPU oracle of the routed MXFP4 MoE layer (test infrastructure only).

Only the tests, the graft entry point's smoke check and bench.py's CPU
baseline import this package; the HIP library never does."""

from .moe import *  # noqa: F401,F403
from . import moe  # noqa: F401
