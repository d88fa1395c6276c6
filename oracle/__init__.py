"""CPU oracle of the MoE FFN forward (fp64).  Test infrastructure only: see moe_oracle."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
from . import backward  # noqa: F401  (fp64 backward, test infrastructure)
