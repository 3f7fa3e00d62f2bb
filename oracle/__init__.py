"""CPU oracle (float64, numpy) for channel-pruned decode attention.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .leank_oracle import *  # noqa: F401,F403
from .leank_oracle import __all__  # noqa: F401
