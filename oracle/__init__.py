"""CPU oracle (test infrastructure only): see ``oracle.brs_oracle``."""
from .brs_oracle import *  # noqa: F401,F403
