"""Exact attention forward and backward for MI355X (gfx950): hand-written HIP kernels behind a C ABI.

``fwd(q, k, v, causal, scale=None, n_split=1) -> (o, lse)`` and ``fwd_out``
call the ``fa_fwd`` / ``fa_fwd_gqa`` / ``fa_fwd_split`` entry points of
``libfa.so`` (declared in ``include/fa.h``); ``fwd_noalloc_out`` calls
``fa_fwd_split_noalloc``, which allocates nothing; ``fwd_fp8`` / ``fwd_fp8_out`` take
FP8 E4M3 inputs and call ``fa_fwd_fp8``; ``bwd(q, k, v, o, lse, do, causal,
scale=None) -> (dq, dk, dv)`` and ``bwd_out`` call ``fa_bwd``.  The library is
loaded on first use; a missing build raises instead of falling back.
``load(variant_path("exp2poly"))`` loads a measurement variant with the same
C ABI, which ``fwd`` / ``fwd_out`` take as ``lib=``.
"""
from ._lib import (FAError, bwd, bwd_out, bwd_workspace_bytes, fwd, fwd_fp8, fwd_fp8_out, fwd_out,  # noqa: F401
                   fwd_noalloc_out, load, split_count, split_workspace_bytes, status_string, variant_path)

__all__ = ["fwd", "fwd_out", "fwd_noalloc_out", "fwd_fp8", "fwd_fp8_out", "bwd", "bwd_out", "bwd_workspace_bytes", "load", "status_string", "split_count",
           "split_workspace_bytes", "variant_path", "FAError"]
