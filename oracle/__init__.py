"""CPU oracle of the AWQ search path -- test infrastructure only.

Imported by the test suite, the smoke check and the benchmark's CPU baseline
leg; never by the product path.
"""
from .awq_oracle import *  # noqa: F401,F403
from . import awq_oracle  # noqa: F401
