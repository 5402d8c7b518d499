"""CPU oracle (test infrastructure only; see sq_oracle's header)."""
from .sq_oracle import *  # noqa: F401,F403
from . import sq_oracle  # noqa: F401
