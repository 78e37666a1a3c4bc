"""CPU oracle for the ZeRO sharded update: test infrastructure only.

Nothing in the product package imports this package, and this package imports
nothing from the product package.
"""
from .zero_oracle import *  # noqa: F401,F403
from . import compare  # noqa: F401
