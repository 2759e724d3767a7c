"""CPU oracle of the routed-expert MoE layer (test infrastructure only)."""
from .moe_oracle import *  # noqa: F401,F403
