"""CPU oracle (test infrastructure only; see svdq_ref's header)."""
from .svdq_ref import *  # noqa: F401,F403
from .svdq_ref import INT4, FP4, GROUP, QMAX  # noqa: F401
