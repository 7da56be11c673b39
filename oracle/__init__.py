"""CPU oracle of the one-GPU MoE layer (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import build_oracle  # noqa: F401
