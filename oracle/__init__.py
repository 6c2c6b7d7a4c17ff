"""CPU oracle (test infrastructure only; see ``nvfp4_oracle``)."""
from .nvfp4_oracle import *  # noqa: F401,F403
from . import nvfp4_oracle  # noqa: F401
