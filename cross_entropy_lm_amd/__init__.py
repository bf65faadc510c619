"""Fused linear log-prob (linear_logp / fused linear cross-entropy) for AMD MI355X.

The computation lives in the HIP library ``libllp.so`` (C ABI in
``include/llp.h``); ``cross_entropy_lm_amd.llp`` is its ctypes binding. The
library is loaded on the first call, not at import.
"""

from . import llp  # noqa: F401

__all__ = ["llp"]
