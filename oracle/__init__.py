"""CPU oracle of the MoE-layer forward (test infrastructure only; see
moe_oracle's module docstring).  Nothing in the product path imports it."""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
