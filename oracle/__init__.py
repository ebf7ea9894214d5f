"""CPU fp64 oracle for the CSA2 layer hot path.

This package is test infrastructure. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it; the
HIP library and its Python binding never do. It shares no code with the GPU
path.
"""

from . import formats  # noqa: F401
from .csa2_oracle import *  # noqa: F401,F403
