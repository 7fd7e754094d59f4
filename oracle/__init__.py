"""CPU oracle of the SmoothQuant W8A8 linear layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, links or runs anything here, and this package imports nothing from it.
"""
from .sq_oracle import *  # noqa: F401,F403
