"""Test infrastructure: the float64 CPU oracle for LRKV decode and append.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import this
package; the library in factored_rank_kv_amd/ never does.
"""
from .lrkv_oracle import *  # noqa: F401,F403
from .lrkv_oracle import Layout, F32, BF16  # noqa: F401
