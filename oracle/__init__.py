"""Float64 CPU oracle for block-sparse prefill attention with mean correction.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path
(the HIP library and its Python binding) never does.
"""
from .fp2_oracle import *  # noqa: F401,F403
from .fp2_oracle import __all__  # noqa: F401
