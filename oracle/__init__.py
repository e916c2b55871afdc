"""TriAttention oracle (test infrastructure only; see triattn_oracle.py)."""
from .triattn_oracle import *  # noqa: F401,F403
from .triattn_oracle import OFFSETS  # noqa: F401
