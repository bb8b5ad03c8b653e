"""MI355X-native MLA speculative-decoding verify attention.

The compute path is the C-ABI library ``libmla_verify.so`` (hand-written HIP
kernels for gfx950) declared in ``include/mla_verify.h``; ``binding`` wraps
it with ctypes over torch device tensors. Importing this package does not
load the library; the first call into ``binding`` does, and raises if the
library is missing (there is no fallback).
"""

__all__ = ["binding", "inputs", "roofline"]
