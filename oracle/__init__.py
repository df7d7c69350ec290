"""fp64 CPU oracle (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the HIP product path never does.
"""
from .taylor_oracle import *  # noqa: F401,F403
from .taylor_oracle import alpha_vector  # noqa: F401
