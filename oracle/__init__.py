"""FP64 CPU oracle (test infrastructure only; never used by the product path)."""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
