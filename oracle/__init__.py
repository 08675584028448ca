"""CPU oracle (fp64, numpy) for the DeepSeek-V4 hybrid attention core.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the benchmark's
CPU-baseline leg.  The HIP library and its Python binding never import it.
"""
from .dsv4_oracle import *  # noqa: F401,F403
from . import dsv4_oracle  # noqa: F401
