"""CPU oracle of the sparse-attention hot path.  TEST INFRASTRUCTURE ONLY.

Importable only from tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg.  Shares no code with the HIP library.
"""
from . import rtp_oracle
from .problem import Problem, from_inputs
