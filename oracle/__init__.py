"""CPU oracle for the POP channel-pruned gated-MLP path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The device path (the HIP library and
its Python binding) never imports, calls or falls back to anything here, and
this package imports nothing from the device path.
"""
from .pop_oracle import *  # noqa: F401,F403
from . import layer_oracle as layer  # noqa: E402,F401  (decoder layer around the pruned FFN)
