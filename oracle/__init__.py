"""CPU oracle for the heterogeneous multi-LoRA linear (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg, never by the product path.  See mlora_oracle.py.
"""
from .mlora_oracle import *  # noqa: F401,F403
from .mlora_oracle import __all__  # noqa: F401
