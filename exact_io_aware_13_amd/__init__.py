"""Exact attention forward for MI355X (gfx950): hand-written HIP kernels behind a C ABI.

``fwd(q, k, v, causal, scale=None, n_split=1) -> (o, lse)`` and ``fwd_out``
call the ``fa_fwd`` / ``fa_fwd_gqa`` / ``fa_fwd_split`` entry points of
``libfa.so`` (declared in ``include/fa.h``).  The library is loaded on first
use; a missing build raises instead of falling back.
"""
from ._lib import (FAError, fwd, fwd_out, load, split_count, split_workspace_bytes,  # noqa: F401
                   status_string)

__all__ = ["fwd", "fwd_out", "load", "status_string", "split_count", "split_workspace_bytes", "FAError"]
