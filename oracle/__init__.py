"""CPU fp64 oracle for the grouped-query-attention block.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library or its binding.
"""
from .gqa_oracle import *  # noqa: F401,F403
