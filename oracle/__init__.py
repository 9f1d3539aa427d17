"""CPU oracle for the partial channel-reduce (test infrastructure only; see pcr_oracle)."""
from .pcr_oracle import *  # noqa: F401,F403
from .pcr_oracle import __all__  # noqa: F401
