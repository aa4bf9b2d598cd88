"""Attention-matching KV compaction on MI355X (gfx950).

The compute path is the C-ABI library ``libamc.so`` (hand-written HIP
kernels); :mod:`attention_matching_least_amd.amc` is its ctypes binding.
Nothing is loaded at import time; the first call into the binding loads the
library and raises if it has not been built.
"""
__all__ = ["amc"]
