"""CPU FP64 oracle (test infrastructure only; never imported by the GPU path)."""
from .flp_oracle import *  # noqa: F401,F403
