"""CPU oracle of the GPTQ layer-quantization pass (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The product path (the HIP library and its binding) never does.
"""
from .gptq_ref import *  # noqa: F401,F403
from .gptq_ref import NotPositiveDefinite  # noqa: F401
