"""fp64 CPU oracle for paged attention and paged block copy.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.
"""
from .paged_attn_oracle import *  # noqa: F401,F403
from .paged_attn_oracle import __all__  # noqa: F401
