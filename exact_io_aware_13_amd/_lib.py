"""ctypes binding of ``libfa.so`` (the C ABI in ``include/fa.h``).

Argument marshalling only: every step of the attention forward and backward
runs in the HIP kernels.  torch supplies device memory and the current HIP stream.  If the
library has not been built, loading fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

# fa_status codes, as in include/fa.h
FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEAD_DIM = 3
FA_ERR_SCALE = 4
FA_ERR_ALIGN = 5
FA_ERR_OVERFLOW = 6
FA_ERR_HIP = 7
FA_ERR_ARG = 8
FA_ERR_SCRATCH = 9
SCRATCH_BYTES = 16 << 20      # FA_SCRATCH_BYTES: the fixed scratch of fa_fwd_split_noalloc

EXPORTED = ("fa_fwd", "fa_fwd_gqa", "fa_fwd_split", "fa_fwd_split_noalloc", "fa_fwd_split_workspace_bytes", "fa_fwd_split_count",
            "fa_fwd_fp8", "fa_fwd_fp8_split", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string", "fa_hip_error_string")

_libs = {}


def variant_path(name: str) -> str:
    """Path of a measurement variant of the library (``libfa_<name>.so``, built by ``build.build_all``)."""
    return os.path.join(_PKG, f"libfa_{name}.so")


class FAError(RuntimeError):
    def __init__(self, status: int, message: str, entry: str = "fa_fwd"):
        super().__init__(f"{entry} failed with status {status}: {message}")
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Load ``libfa.so``, or the library at ``path`` (a measurement variant with
    the same C ABI); raises if it is missing."""
    path = path or LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                               "(or python exact_io_aware_13_amd/build.py) first")
        lib = ctypes.CDLL(path)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp]
        lib.fa_fwd.restype = ctypes.c_int
        lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp]
        lib.fa_fwd_gqa.restype = ctypes.c_int
        lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_float, i64, vp, ctypes.c_size_t, vp]
        lib.fa_fwd_split.restype = ctypes.c_int
        lib.fa_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                             ctypes.c_float, i64, vp]
        lib.fa_fwd_split_noalloc.restype = ctypes.c_int
        lib.fa_fwd_split_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
        lib.fa_fwd_split_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_split_count.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
        lib.fa_fwd_split_count.restype = ctypes.c_int64
        f32 = ctypes.c_float
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int, f32, f32, f32,
                                   f32, vp]
        lib.fa_fwd_fp8.restype = ctypes.c_int
        lib.fa_fwd_fp8_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int, f32, f32, f32,
                                         f32, i64, vp, ctypes.c_size_t, vp]
        lib.fa_fwd_fp8_split.restype = ctypes.c_int
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                               ctypes.c_float, vp, ctypes.c_size_t, vp]
        lib.fa_bwd.restype = ctypes.c_int
        lib.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_status_string.argtypes = [ctypes.c_int]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_hip_error_string.argtypes = []
        lib.fa_hip_error_string.restype = ctypes.c_char_p
        _libs[path] = lib
    return _libs[path]


def status_string(status: int, lib: ctypes.CDLL | None = None) -> str:
    return (lib or load()).fa_status_string(int(status)).decode()


def fa_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
               B: int, H: int, T: int, d: int, causal: int, scale: float, stream: int,
               lib: ctypes.CDLL | None = None) -> int:
    """Call ``fa_fwd`` with raw addresses; returns the fa_status code."""
    return int((lib or load()).fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, T, d, int(causal),
                                      float(scale), stream))


def fa_fwd_gqa_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, Hq: int, Hkv: int,
                   T: int, d: int, causal: int, scale: float, stream: int, lib: ctypes.CDLL | None = None) -> int:
    """Call ``fa_fwd_gqa`` with raw addresses; returns the fa_status code."""
    return int((lib or load()).fa_fwd_gqa(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, T, d, int(causal),
                                          float(scale), stream))


def fa_fwd_split_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, Hq: int, Hkv: int,
                     Tq: int, Tk: int, d: int, causal: int, scale: float, n_split: int, ws_ptr: int,
                     ws_bytes: int, stream: int, lib: ctypes.CDLL | None = None) -> int:
    """Call ``fa_fwd_split`` with raw addresses; returns the fa_status code."""
    return int((lib or load()).fa_fwd_split(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Tq, Tk, d,
                                            int(causal), float(scale), n_split, ws_ptr, ws_bytes, stream))


def fa_fwd_split_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, Hq: int,
                             Hkv: int, Tq: int, Tk: int, d: int, causal: int, scale: float, n_split: int,
                             stream: int) -> int:
    """Call ``fa_fwd_split_noalloc`` with raw addresses; returns the fa_status code."""
    return int(load().fa_fwd_split_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Tq, Tk, d,
                                           int(causal), float(scale), int(n_split), stream))


def split_workspace_bytes(B: int, Hq: int, Tq: int, Tk: int, d: int, n_split: int,
                          lib: ctypes.CDLL | None = None) -> int:
    return int((lib or load()).fa_fwd_split_workspace_bytes(B, Hq, Tq, Tk, d, n_split))


def split_count(B: int, Hq: int, Hkv: int, Tq: int, Tk: int, d: int, causal: bool,
                lib: ctypes.CDLL | None = None) -> int:
    return int((lib or load()).fa_fwd_split_count(B, Hq, Hkv, Tq, Tk, d, int(bool(causal))))


def fa_fwd_fp8_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, Hq: int, Hkv: int,
                   Tq: int, Tk: int, d: int, causal: int, scale: float, q_descale: float, k_descale: float,
                   v_descale: float, stream: int) -> int:
    """Call ``fa_fwd_fp8`` with raw addresses; returns the fa_status code."""
    return int(load().fa_fwd_fp8(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Tq, Tk, d, int(causal),
                                 float(scale), float(q_descale), float(k_descale), float(v_descale), stream))


def fa_fwd_fp8_split_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, Hq: int, Hkv: int,
                         Tq: int, Tk: int, d: int, causal: int, scale: float, q_descale: float, k_descale: float,
                         v_descale: float, n_split: int, ws_ptr: int, ws_bytes: int, stream: int) -> int:
    """Call ``fa_fwd_fp8_split`` with raw addresses; returns the fa_status code."""
    return int(load().fa_fwd_fp8_split(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Tq, Tk, d, int(causal),
                                       float(scale), float(q_descale), float(k_descale), float(v_descale),
                                       int(n_split), ws_ptr, ws_bytes, stream))


def fa_bwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, do_ptr: int, lse_ptr: int, dq_ptr: int,
               dk_ptr: int, dv_ptr: int, B: int, Hq: int, Hkv: int, Tq: int, Tk: int, d: int, causal: int,
               scale: float, ws_ptr: int, ws_bytes: int, stream: int) -> int:
    """Call ``fa_bwd`` with raw addresses; returns the fa_status code."""
    return int(load().fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, B, Hq, Hkv, Tq,
                             Tk, d, int(causal), float(scale), ws_ptr, ws_bytes, stream))


def bwd_workspace_bytes(B: int, Hq: int, Tq: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, Hq, Tq))


def _check(status: int, entry: str = "fa_fwd", lib: ctypes.CDLL | None = None) -> None:
    if status != FA_OK:
        msg = status_string(status, lib)
        if status == FA_ERR_HIP:
            msg += f" ({(lib or load()).fa_hip_error_string().decode()})"
        raise FAError(status, msg, entry)


def _check_tensors(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must have shape (B, H, T, d), got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape:
        raise ValueError(f"k, v shapes differ: {tuple(k.shape)}, {tuple(v.shape)}")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError(f"q {tuple(q.shape)} and k/v {tuple(k.shape)} differ in batch or head size")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def _check_workspace(workspace, device) -> None:
    """A caller's workspace must be one contiguous GPU tensor on ``device`` (its bytes are passed raw)."""
    import torch
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")


def fwd_out(q, k, v, o, lse, causal: bool, scale: float | None = None, n_split: int | None = 1,
            workspace=None, lib: ctypes.CDLL | None = None) -> None:
    """Exact attention forward into caller buffers ``o`` (bf16, like q) and ``lse`` (fp32, (B, Hq, Tq)).

    ``q``: (B, Hq, Tq, d); ``k, v``: (B, Hkv, Tk, d).  One key/value head per
    query head with Tq == Tk and one split calls ``fa_fwd``; grouped heads call
    ``fa_fwd_gqa``; anything else (Tq != Tk, or ``n_split`` != 1; ``None`` asks
    the library for a split count) calls ``fa_fwd_split``.  A split forward
    needs ``workspace`` (a uint8 GPU tensor of ``split_workspace_bytes`` bytes);
    if it is not given, one is allocated here.  ``lib``: a library from
    ``load(path)`` (a measurement variant) instead of ``libfa.so``.
    """
    import torch
    _check_tensors(q, k, v)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous bf16 tensor shaped like q on q's device")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, Tq) on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_split is None:
        n_split = split_count(B, Hq, Hkv, Tq, Tk, d, causal, lib)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if Tq == Tk and n_split == 1:
            if Hkv == Hq:
                st = fa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, Hq, Tq, d, int(bool(causal)), float(scale), stream, lib)
            else:
                st = fa_fwd_gqa_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    B, Hq, Hkv, Tq, d, int(bool(causal)), float(scale), stream, lib)
        else:
            need = split_workspace_bytes(B, Hq, Tq, Tk, d, n_split, lib)
            if workspace is None and need > 0:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            elif workspace is not None:
                _check_workspace(workspace, q.device)
            ws_ptr = workspace.data_ptr() if workspace is not None else 0
            ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
            st = fa_fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, Hq, Hkv, Tq, Tk, d, int(bool(causal)), float(scale), int(n_split),
                                  ws_ptr, ws_bytes, stream, lib)
        _check(st, "fa_fwd", lib)


def fwd_noalloc_out(q, k, v, o, lse, causal: bool, scale: float | None = None, n_split: int | None = None) -> None:
    """``fwd_out`` with split keys through ``fa_fwd_split_noalloc``: no memory is
    allocated, by the library or here; the partial results go to the library's
    fixed per-GPU scratch (``SCRATCH_BYTES``).  Calls that overlap on one GPU
    race on that scratch.  ``n_split=None`` asks the library for a split count."""
    import torch
    _check_tensors(q, k, v)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous bf16 tensor shaped like q on q's device")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, Tq) on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_split is None:
        n_split = split_count(B, Hq, Hkv, Tq, Tk, d, causal)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_fwd_split_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      B, Hq, Hkv, Tq, Tk, d, int(bool(causal)), float(scale), int(n_split), stream)
    _check(st, "fa_fwd_split_noalloc")


def fwd(q, k, v, causal: bool, scale: float | None = None, n_split: int | None = 1,
        lib: ctypes.CDLL | None = None):
    """Exact attention forward; returns ``(o, lse)``.

    ``q``: contiguous bf16 GPU tensor (B, Hq, Tq, d); ``k, v``: (B, Hkv, Tk, d),
    d in {64, 128}, Hq a multiple of Hkv.  ``scale`` defaults to 1/sqrt(d).
    With ``causal`` the queries are the last Tq positions (query i sees keys
    j <= i + Tk - Tq).  ``o`` is bf16 like ``q``; ``lse`` is float32
    (B, Hq, Tq) in natural-log units.  ``n_split`` and ``lib`` as in ``fwd_out``.
    """
    import torch
    _check_tensors(q, k, v)
    B, Hq, Tq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    fwd_out(q, k, v, o, lse, causal, scale, n_split, lib=lib)
    return o, lse


def _check_fp8_tensors(q, k, v):
    import torch
    fp8 = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in fp8:
            raise ValueError(f"{name} must hold E4M3 bytes (uint8 or float8_e4m3fn), got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous (B, H, T, d) tensor, got {tuple(t.shape)}")
    if k.shape != v.shape:
        raise ValueError(f"k, v shapes differ: {tuple(k.shape)}, {tuple(v.shape)}")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError(f"q {tuple(q.shape)} and k/v {tuple(k.shape)} differ in batch or head size")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def fwd_fp8_out(q, k, v, o, lse, causal: bool, scale: float | None = None, descales=(1.0, 1.0, 1.0),
                n_split: int | None = 1, workspace=None) -> None:
    """FP8 forward into caller buffers ``o`` (bf16, shaped like q) and ``lse`` (fp32, (B, Hq, Tq)).

    ``q``: (B, Hq, Tq, d), ``k, v``: (B, Hkv, Tk, d), E4M3 bytes (uint8 or
    float8_e4m3fn); ``descales`` = (q_descale, k_descale, v_descale), the
    operands being ``descale * e4m3``.  ``n_split`` = 1 calls ``fa_fwd_fp8``;
    otherwise ``fa_fwd_fp8_split`` with a workspace as for ``fwd_out`` (``None``
    asks the library for a split count; a workspace is allocated here if not
    given).
    """
    import torch
    _check_fp8_tensors(q, k, v)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous bf16 tensor shaped like q on q's device")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, Tq) on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qd, kd, vd = (float(x) for x in descales)
    if n_split is None:
        n_split = split_count(B, Hq, Hkv, Tq, Tk, d, causal)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if n_split == 1:
            st = fa_fwd_fp8_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                                Tq, Tk, d, int(bool(causal)), float(scale), qd, kd, vd, stream)
            _check(st, "fa_fwd_fp8")
            return
        need = split_workspace_bytes(B, Hq, Tq, Tk, d, n_split)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif workspace is not None:
            _check_workspace(workspace, q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else 0
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        st = fa_fwd_fp8_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                                  Tq, Tk, d, int(bool(causal)), float(scale), qd, kd, vd, int(n_split), ws_ptr,
                                  ws_bytes, stream)
        _check(st, "fa_fwd_fp8_split")


def fwd_fp8(q, k, v, causal: bool, scale: float | None = None, descales=(1.0, 1.0, 1.0), n_split: int | None = 1):
    """FP8 E4M3 attention forward; returns ``(o, lse)`` with ``o`` bf16 and
    ``lse`` float32 (B, Hq, Tq).  Arguments as ``fwd_fp8_out``."""
    import torch
    _check_fp8_tensors(q, k, v)
    B, Hq, Tq, d = q.shape
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    fwd_fp8_out(q, k, v, o, lse, causal, scale, descales, n_split)
    return o, lse


def bwd_out(q, k, v, o, lse, do, dq, dk, dv, causal: bool, scale: float | None = None, workspace=None) -> None:
    """Gradients of the forward into caller buffers ``dq`` (like q), ``dk``, ``dv`` (like k, v).

    ``o`` and ``lse`` are the forward's outputs for the same q, k, v, causal
    and scale; ``do`` is the upstream gradient of o (bf16, shaped like q).
    ``workspace`` is a uint8 GPU tensor of at least ``bwd_workspace_bytes``
    bytes; if it is not given, one is allocated here.
    """
    import torch
    _check_tensors(q, k, v)
    B, Hq, Tq, d = q.shape
    for name, t, like in (("o", o, q), ("do", do, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if (not isinstance(t, torch.Tensor) or t.shape != like.shape or t.dtype != torch.bfloat16
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped {tuple(like.shape)} on q's device")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, Tq) on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = bwd_workspace_bytes(B, Hq, Tq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, k.shape[1], Tq, k.shape[2], d,
                        int(bool(causal)), float(scale), workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), stream)
        _check(st, "fa_bwd")


def bwd(q, k, v, o, lse, do, causal: bool, scale: float | None = None):
    """Gradients of the exact attention forward; returns ``(dq, dk, dv)`` (bf16)."""
    import torch
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    bwd_out(q, k, v, o, lse, do, dq, dk, dv, causal, scale)
    return dq, dk, dv
