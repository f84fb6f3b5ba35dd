"""CPU oracle for the W4A16 MoE expert GEMM pair -- test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path.
"""
from .qma_oracle import *  # noqa: F401,F403
