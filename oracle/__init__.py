"""Plain, slow CPU oracle of the Stem prefill path.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.  The
library's product path never calls it, and it imports nothing from the library or its kernels.
"""
from .stem_oracle import *  # noqa: F401,F403
from .stem_oracle import __all__  # noqa: F401
