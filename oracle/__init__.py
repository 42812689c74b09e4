"""fp64 CPU oracle for the MLA hot path.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  The product path never does.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import __all__  # noqa: F401
