"""CPU oracle package (test infrastructure; see moe_oracle's header)."""
from .moe_oracle import *  # noqa: F401,F403
