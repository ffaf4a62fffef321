"""CPU oracle (test infrastructure only; see mxfp4_oracle.py)."""
from .mxfp4_oracle import *  # noqa: F401,F403
from . import mxfp4_oracle  # noqa: F401
