"""CPU oracle (test infrastructure only; see kvq_oracle.py's header)."""
from .kvq_oracle import *  # noqa: F401,F403
from .kvq_oracle import WHT_C  # noqa: F401
