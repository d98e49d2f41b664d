"""CPU oracle for BLASST skip-softmax attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU path.
"""
from .blasst_oracle import *  # noqa: F401,F403
from .blasst_oracle import __all__  # noqa: F401
