"""Float64 CPU oracle for the chunkwise KDA forward (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may use
this package. The HIP library never imports, links or calls it.
"""
from .kda_oracle import *  # noqa: F401,F403
