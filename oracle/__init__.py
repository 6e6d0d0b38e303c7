"""CPU oracle for the exact attention forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
(``exact_io_aware_13_amd``) never imports it, and the two share no code.

Contents
--------
* ``attention_f64`` / ``attention_rows_f64``: ctypes wrappers around the plain
  C oracle in ``fa_ref.c`` (fp64, one row at a time, OpenMP over rows).  This
  is the definition the method must reproduce: ordinary softmax attention with
  the causal rule of "Flash Attention, tiled: exact attention without the T x T
  HBM matrix" (section "Ordinary causal attention").
* ``attention_bwd_f64`` / ``attention_bwd_rows_f64``: the gradients of the same
  attention with respect to Q, K and V for an upstream gradient dO (fp64, the
  chain rule through the softmax one row at a time), the backward that
  "FlashAttention and Fused Kernels: Attention Without the n x n Matrix"
  ("Training: recompute instead of store") describes.
* ``widen_bf16``: exact widening of bf16 bit patterns to float64, so that the
  oracle consumes the very values the GPU receives.
* ``online`` (submodule): the online-softmax recurrence, tile by tile, used to
  check that the recurrence and the definition agree.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_ref.c")
_LIB = os.path.join(_HERE, "libfa_ref.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``fa_ref.c`` into ``libfa_ref.so`` with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.fa_ref_fwd_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int,
                                       ctypes.c_double]
        lib.fa_ref_fwd_f64.restype = ctypes.c_int
        lib.fa_ref_fwd_rows_f64.argtypes = [dp, dp, dp, i64, i64, i64, i64, ctypes.c_int,
                                            ctypes.c_double, ctypes.POINTER(ctypes.c_int64), i64,
                                            dp, dp]
        lib.fa_ref_fwd_rows_f64.restype = ctypes.c_int
        lib.fa_ref_attn_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                        ctypes.c_double]
        lib.fa_ref_attn_f64.restype = ctypes.c_int
        lib.fa_ref_attn_rows_f64.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                             ctypes.c_double, ctypes.POINTER(ctypes.c_int64), i64, dp, dp]
        lib.fa_ref_attn_rows_f64.restype = ctypes.c_int
        lib.fa_ref_attn_bwd_f64.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                            ctypes.c_double, dp, dp, dp]
        lib.fa_ref_attn_bwd_f64.restype = ctypes.c_int
        ip = ctypes.POINTER(ctypes.c_int64)
        lib.fa_ref_attn_bwd_rows_f64.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                                 ctypes.c_double, ip, i64, dp, ip, i64, dp, dp]
        lib.fa_ref_attn_bwd_rows_f64.restype = ctypes.c_int
        lib.fa_ref_attn_bwd_rows_given_d_f64.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                                         ctypes.c_double, dp, ip, i64, dp, ip, i64, dp, dp]
        lib.fa_ref_attn_bwd_rows_given_d_f64.restype = ctypes.c_int
        lib.fa_ref_num_threads.argtypes = []
        lib.fa_ref_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of an fp32)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return np.ascontiguousarray(x, dtype=np.float64)


def _check4(q, k, v):
    """q: (B, Hq, Tq, d); k, v: (B, Hkv, Tk, d) with Hq a multiple of Hkv."""
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError(f"q must be (B, Hq, Tq, d) and k, v one (B, Hkv, Tk, d) shape; got "
                         f"{q.shape}, {k.shape}, {v.shape}")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3] or q.shape[1] % k.shape[1] != 0:
        raise ValueError(f"incompatible q {q.shape} and k/v {k.shape}")


def attention_f64(q, k, v, causal: bool, scale: float):
    """Exact attention forward over every row.

    ``q``: (B, Hq, Tq, d); ``k, v``: (B, Hkv, Tk, d), Hq a multiple of Hkv
    (query head h reads key/value head h // (Hq // Hkv)); either float64/float32
    values or uint16 bf16 bit patterns (widened exactly).  With ``causal`` the
    queries are the last Tq positions: query i sees keys j <= i + Tk - Tq.
    Returns ``(o, lse)`` as float64 with shapes (B, Hq, Tq, d) and (B, Hq, Tq);
    ``lse`` is in natural-log units.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check4(q, k, v)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    o = np.empty((B, Hq, Tq, d), dtype=np.float64)
    lse = np.empty((B, Hq, Tq), dtype=np.float64)
    rc = _load().fa_ref_attn_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse),
                                 B, Hq, Hkv, Tq, Tk, d, int(bool(causal)), float(scale))
    if rc != 0:
        raise RuntimeError(f"fa_ref_attn_f64 failed with code {rc}")
    return o, lse


def attention_rows_f64(q, k, v, causal: bool, scale: float, rows):
    """Exact attention forward for selected rows only.

    Shapes and rules as ``attention_f64``; ``rows`` holds flat row indices
    ``(b*Hq + h)*Tq + i``.  Returns ``(o_rows, lse_rows)`` with shapes (n, d)
    and (n,).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check4(q, k, v)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().fa_ref_attn_rows_f64(_dptr(q), _dptr(k), _dptr(v), B, Hq, Hkv, Tq, Tk, d,
                                      int(bool(causal)), float(scale),
                                      rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n,
                                      _dptr(o), _dptr(lse))
    if rc != 0:
        raise RuntimeError(f"fa_ref_attn_rows_f64 failed with code {rc}")
    return o, lse


def attention_bwd_f64(q, k, v, do, causal: bool, scale: float):
    """Gradients of the exact attention forward.

    ``q``, ``do``: (B, Hq, Tq, d); ``k``, ``v``: (B, Hkv, Tk, d) (values or
    bf16 bit patterns, as ``attention_f64``).  Returns ``(dq, dk, dv)`` in
    float64 with the shapes of ``q``, ``k``, ``v``; dk and dv of a key/value
    head sum the contributions of every query head of its group.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    _check4(q, k, v)
    if do.shape != q.shape:
        raise ValueError(f"do must have the shape of q {q.shape}; got {do.shape}")
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _load().fa_ref_attn_bwd_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(do), B, Hq, Hkv, Tq, Tk, d,
                                     int(bool(causal)), float(scale), _dptr(dq), _dptr(dk), _dptr(dv))
    if rc != 0:
        raise RuntimeError(f"fa_ref_attn_bwd_f64 failed with code {rc}")
    return dq, dk, dv


def attention_bwd_rows_f64(q, k, v, do, causal: bool, scale: float, qrows, krows, d_rows=None):
    """Selected gradient rows: dq for flat query rows ``(b*Hq + h)*Tq + i`` and
    dk, dv for flat key rows ``(b*Hkv + hk)*Tk + j``.  Returns
    ``(dq_rows, dk_rows, dv_rows)`` of shapes (len(qrows), d) and (len(krows), d).

    ``d_rows`` (optional, float64 of shape (B, Hq, Tq)) replaces the softmax
    Jacobian term D_i = sum_j P_ij dP_ij of every row; only the rows that the
    requested gradients depend on are read."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    _check4(q, k, v)
    if do.shape != q.shape:
        raise ValueError(f"do must have the shape of q {q.shape}; got {do.shape}")
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    qrows = np.ascontiguousarray(qrows, dtype=np.int64)
    krows = np.ascontiguousarray(krows, dtype=np.int64)
    dq = np.empty((qrows.shape[0], d), dtype=np.float64)
    dk = np.empty((krows.shape[0], d), dtype=np.float64)
    dv = np.empty((krows.shape[0], d), dtype=np.float64)
    ip = ctypes.POINTER(ctypes.c_int64)
    if d_rows is None:
        dptr = ctypes.cast(None, ctypes.POINTER(ctypes.c_double))
    else:
        d_rows = np.ascontiguousarray(d_rows, dtype=np.float64)
        if d_rows.shape != (B, Hq, Tq):
            raise ValueError(f"d_rows must have shape {(B, Hq, Tq)}; got {d_rows.shape}")
        dptr = _dptr(d_rows)
    rc = _load().fa_ref_attn_bwd_rows_given_d_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(do), B, Hq, Hkv, Tq, Tk, d,
                                                  int(bool(causal)), float(scale), dptr,
                                                  qrows.ctypes.data_as(ip), qrows.shape[0], _dptr(dq),
                                                  krows.ctypes.data_as(ip), krows.shape[0], _dptr(dk), _dptr(dv))
    if rc != 0:
        raise RuntimeError(f"fa_ref_attn_bwd_rows_f64 failed with code {rc}")
    return dq, dk, dv


def num_threads() -> int:
    """OpenMP threads the C oracle uses (OMP_NUM_THREADS, else all host cores)."""
    return int(_load().fa_ref_num_threads())
