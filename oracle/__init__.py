"""CPU oracle for LoopVQ (test infrastructure only; see loopvq_oracle.py)."""
from .loopvq_oracle import *  # noqa: F401,F403
from . import loopvq_oracle as ref  # noqa: F401
