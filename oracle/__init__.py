"""CPU oracle for the paged-KV attention step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the build entry point's smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports, calls or links it.
"""
from .pa_oracle import *  # noqa: F401,F403
from .pa_oracle import __all__  # noqa: F401
