"""CPU oracle for the LLM.int8() linear layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product never does.
"""
from .llm_int8 import *  # noqa: F401,F403
from .llm_int8 import ulp16  # noqa: F401
