"""Exact attention forward for MI355X (gfx950): hand-written HIP kernels behind a C ABI.

``fwd(q, k, v, causal, scale=None) -> (o, lse)`` and ``fwd_out`` call the
``fa_fwd`` entry point of ``libfa.so`` (declared in ``include/fa.h``).  The
library is loaded on first use; a missing build raises instead of falling back.
"""
from ._lib import FAError, fwd, fwd_out, load, status_string  # noqa: F401

__all__ = ["fwd", "fwd_out", "load", "status_string", "FAError"]
