"""Float64 CPU oracle for attention-matching KV compaction.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline may import it; the library and its Python binding never do.
"""
from .amc_oracle import *  # noqa: F401,F403
from . import amc_oracle  # noqa: F401
