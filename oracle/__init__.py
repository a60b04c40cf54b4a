"""f64 CPU oracle for block-quantized GEMV (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""
from .oracle import *  # noqa: F401,F403
from .oracle import build  # noqa: F401
