"""fp64 CPU oracle of the MoE expert layer (test infrastructure only; the
product path never imports it)."""
from .moe_oracle import *  # noqa: F401,F403
