"""CPU oracle (test infrastructure only; see ``oracle.wq_oracle``)."""
from .wq_oracle import *  # noqa: F401,F403
from .wq_oracle import __all__  # noqa: F401
