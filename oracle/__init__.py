"""fp64 CPU oracle of the QSA layer forward pass.

TEST INFRASTRUCTURE: imported only by tests/, by the package's smoke check and
by the CPU-baseline leg of bench.py.  It shares no code with the HIP library
or its binding, and imports nothing from them.
"""
from .qsa_oracle import *  # noqa: F401,F403
