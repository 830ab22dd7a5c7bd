"""CPU fp64 oracle of the TTT-E2E inner loop (test infrastructure only)."""
from .ttt_oracle import *  # noqa: F401,F403
from .ttt_oracle import Oracle, prefill  # noqa: F401
