"""The C ABI library, on the host: it loads, exports every function that
include/*.h declares, and rejects invalid arguments before any HIP call
(so these run without a GPU).  No attention is computed here."""
import ctypes
import glob
import math
import os
import re
import subprocess

import pytest

from exact_io_aware_13_amd import _lib
from exact_io_aware_13_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from exact_io_aware_13_amd import build
        build.build(force=True)
    return _lib.load()


def test_header_declares_expected_entry_points():
    assert _declared_functions() == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


@pytest.mark.parametrize("name", sorted(build_mod.VARIANTS))
def test_variant_library_exports_every_declared_symbol(name):
    """Each measurement variant is the same C ABI built with one compile-time choice changed."""
    path = _lib.variant_path(name)
    assert path == build_mod.variant_path(name)
    if not os.path.exists(path):
        build_mod.build(force=True, extra=build_mod.VARIANTS[name], out=path)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert _declared_functions() <= exported
    vlib = _lib.load(path)
    assert vlib is not _lib.load() and vlib is _lib.load(path)
    assert _lib.status_string(0, vlib) == _lib.status_string(0)


def test_status_strings(lib):
    for code in range(0, 10):
        s = _lib.status_string(code)
        assert s and s != "unknown status"
    assert _lib.status_string(99) == "unknown status"
    assert lib.fa_hip_error_string() == b""


# Fake, never-dereferenced addresses: validation must fail before any HIP call.
A = 1 << 20


def call(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, T=16, d=64, causal=1, scale=0.125):
    return _lib.fa_fwd_raw(q, k, v, o, lse, B, H, T, d, causal, scale, 0)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_null_pointer(lib, which):
    assert call(**{which: 0}) == _lib.FA_ERR_NULL


@pytest.mark.parametrize("B,H,T", [(0, 1, 1), (1, 0, 1), (1, 1, 0), (-1, 1, 1), (1, 1, -5)])
def test_bad_shape(lib, B, H, T):
    assert call(B=B, H=H, T=T) == _lib.FA_ERR_SHAPE


@pytest.mark.parametrize("d", [0, 1, 32, 63, 65, 96, 127, 129, 256])
def test_bad_head_dim(lib, d):
    assert call(d=d) == _lib.FA_ERR_HEAD_DIM


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf, 3e38, -3e38])
def test_bad_scale(lib, scale):
    assert call(scale=scale) == _lib.FA_ERR_SCALE


@pytest.mark.parametrize("causal", [-1, 2, 7])
def test_bad_causal(lib, causal):
    assert call(causal=causal) == _lib.FA_ERR_ARG


@pytest.mark.parametrize("which,off", [("q", 2), ("k", 8), ("v", 4), ("o", 1), ("lse", 2)])
def test_misaligned(lib, which, off):
    kw = {"q": A, "k": 2 * A, "v": 3 * A, "o": 4 * A, "lse": 5 * A}
    kw[which] += off
    assert call(**kw) == _lib.FA_ERR_ALIGN


def test_overflow(lib):
    assert call(B=1 << 40, H=1 << 30, T=1 << 10) == _lib.FA_ERR_OVERFLOW
    assert call(B=1, H=1, T=(1 << 31) - 1) == _lib.FA_ERR_OVERFLOW
    assert call(B=1 << 20, H=1 << 20, T=1024) == _lib.FA_ERR_OVERFLOW


def test_outputs_overlapping_inputs(lib):
    # o inside q's byte range, lse inside v's, o overlapping lse
    assert call(q=A, o=A + 64, B=1, H=1, T=16, d=64) == _lib.FA_ERR_ARG
    assert call(v=3 * A, lse=3 * A + 16) == _lib.FA_ERR_ARG
    assert call(o=4 * A, lse=4 * A + 1024) == _lib.FA_ERR_ARG


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    import exact_io_aware_13_amd as fa
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x, True)
    with pytest.raises(ValueError):
        fa.fwd(x.float(), x, x, True)


def call_gqa(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, Hq=4, Hkv=2, T=16, d=64, causal=1, scale=0.125):
    return _lib.fa_fwd_gqa_raw(q, k, v, o, lse, B, Hq, Hkv, T, d, causal, scale, 0)


def call_split(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, Hq=4, Hkv=2, Tq=4, Tk=1024, d=64, causal=1,
               scale=0.125, n_split=4, ws=16 * A, ws_bytes=1 << 30):
    return _lib.fa_fwd_split_raw(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, n_split, ws, ws_bytes, 0)


@pytest.mark.parametrize("Hq,Hkv", [(4, 3), (2, 4), (4, 0), (0, 1), (6, 4)])
def test_gqa_bad_head_counts(lib, Hq, Hkv):
    assert call_gqa(Hq=Hq, Hkv=Hkv) == _lib.FA_ERR_SHAPE


def test_gqa_other_checks(lib):
    assert call_gqa(k=0) == _lib.FA_ERR_NULL
    assert call_gqa(d=96) == _lib.FA_ERR_HEAD_DIM
    assert call_gqa(v=3 * A + 8) == _lib.FA_ERR_ALIGN
    assert call_gqa(scale=math.nan) == _lib.FA_ERR_SCALE


def test_split_shape_rules(lib):
    assert call_split(Tq=2048, Tk=1024, causal=1) == _lib.FA_ERR_SHAPE      # causal needs Tq <= Tk
    assert call_split(Tq=0) == _lib.FA_ERR_SHAPE
    assert call_split(Tk=0) == _lib.FA_ERR_SHAPE
    assert call_split(Hq=6, Hkv=4) == _lib.FA_ERR_SHAPE


def test_split_workspace_rules(lib):
    assert call_split(n_split=0) == _lib.FA_ERR_ARG
    assert call_split(n_split=-3) == _lib.FA_ERR_ARG
    assert call_split(ws=0, ws_bytes=0) == _lib.FA_ERR_NULL                  # 4 splits need scratch
    need = _lib.split_workspace_bytes(1, 4, 4, 1024, 64, 4)
    assert call_split(ws_bytes=need - 4) == _lib.FA_ERR_ARG
    assert call_split(ws=16 * A + 4) == _lib.FA_ERR_ALIGN
    assert call_split(ws=A) == _lib.FA_ERR_ARG                               # workspace over q


def call_noalloc(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, Hq=4, Hkv=2, Tq=4, Tk=1024, d=64, causal=1,
                 scale=0.125, n_split=4):
    return _lib.fa_fwd_split_noalloc_raw(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, n_split, 0)


def test_noalloc_validates_before_any_hip_call(lib):
    # every argument check of fa_fwd_split, and then the scratch bound, come before any HIP call
    assert call_noalloc(q=0) == _lib.FA_ERR_NULL
    assert call_noalloc(Tq=2048, Tk=1024) == _lib.FA_ERR_SHAPE
    assert call_noalloc(d=96) == _lib.FA_ERR_HEAD_DIM
    assert call_noalloc(n_split=0) == _lib.FA_ERR_ARG
    assert call_noalloc(scale=float("inf")) == _lib.FA_ERR_SCALE
    assert call_noalloc(o=4 * A + 2) == _lib.FA_ERR_ALIGN
    assert call_noalloc(o=A) == _lib.FA_ERR_ARG                             # o over q
    assert lib.fa_hip_error_string() == b""


def test_noalloc_rejects_splits_beyond_its_scratch(lib):
    # 8 chunks of d = 128 rows take 8 * 129 * 4 bytes per query row: 4064 rows fit in 16 MiB, 4065 do not
    assert _lib.SCRATCH_BYTES == 16 << 20
    fits = _lib.split_workspace_bytes(1, 1, 4064, 8192, 128, 8)
    assert fits <= _lib.SCRATCH_BYTES < _lib.split_workspace_bytes(1, 1, 4065, 8192, 128, 8)
    far = {n: (i + 1) << 32 for i, n in enumerate(("q", "k", "v", "o", "lse"))}   # buffers far apart
    assert call_noalloc(**far, Hq=1, Hkv=1, Tq=4065, Tk=8192, d=128, causal=0, n_split=8) == _lib.FA_ERR_SCRATCH
    assert call_noalloc(**far, B=64, Hq=32, Hkv=8, Tq=1, Tk=32768, d=128, causal=1, n_split=64) == _lib.FA_ERR_SCRATCH
    assert "scratch" in _lib.status_string(_lib.FA_ERR_SCRATCH)
    assert lib.fa_hip_error_string() == b""


def test_split_workspace_bytes(lib):
    # four chunks of 256 keys: 4 x (B Hq Tq) rows x (d + 1) floats
    assert _lib.split_workspace_bytes(1, 4, 4, 1024, 64, 4) == 4 * 16 * 65 * 4
    # chunks round up to whole 64-key tiles: 100 keys in 7 splits is two chunks of 64
    assert _lib.split_workspace_bytes(2, 3, 5, 100, 128, 7) == 2 * (2 * 3 * 5) * 129 * 4
    # one chunk: no workspace
    assert _lib.split_workspace_bytes(1, 1, 1, 64, 64, 8) == 0
    assert _lib.split_workspace_bytes(1, 1, 1, 1000, 64, 1) == 0
    assert _lib.split_workspace_bytes(0, 1, 1, 1000, 64, 2) == 0


def test_grouped_fold_overflow(lib):
    # Grouped heads without the mask fold the group into one head's rows; a row
    # count past 32 bits is rejected before the fold can overflow.
    assert call_gqa(Hq=1 << 40, Hkv=1, T=1 << 30, causal=0) == _lib.FA_ERR_OVERFLOW
    assert call_gqa(Hq=4, Hkv=1, T=(1 << 30) + 1, causal=0) == _lib.FA_ERR_OVERFLOW
    assert call_split(Hq=1 << 62, Hkv=1, Tq=4, Tk=64, causal=0, n_split=1) == _lib.FA_ERR_OVERFLOW
    assert fcall(Hq=1 << 40, Hkv=1, Tq=1 << 30, Tk=1 << 30, causal=0) == _lib.FA_ERR_OVERFLOW
    assert _lib.split_count(1, 1 << 62, 1, 4, 1 << 20, 128, False) == 1
    assert _lib.split_count(1 << 62, 1 << 62, 1 << 62, 1, 1 << 20, 128, True) == 1
    assert lib.fa_hip_error_string() == b""


def test_split_count_advice(lib):
    assert _lib.split_count(1, 32, 32, 1, 32768, 128, True) > 1       # decode: one row per head
    assert _lib.split_count(1, 32, 8, 8192, 8192, 128, True) == 1     # prefill fills the GPU
    assert _lib.split_count(1, 1, 1, 1, 64, 64, False) == 1           # a single tile cannot split
    assert 1 <= _lib.split_count(1, 8, 8, 1, 1 << 20, 64, False) <= 64
    # grouped decode folds the group into rows: fewer workgroups, so more splits
    assert _lib.split_count(8, 32, 8, 1, 32768, 128, True) > _lib.split_count(8, 32, 32, 1, 32768, 128, True)
    assert _lib.split_count(1, 32, 33, 1, 4096, 128, True) == 1       # invalid grouping


# fa_bwd: the same validation before any HIP call.
def bcall(q=A, k=2 * A, v=3 * A, o=4 * A, do=5 * A, lse=6 * A, dq=7 * A, dk=8 * A, dv=9 * A, B=1, Hq=1, Hkv=1,
          Tq=16, Tk=16, d=64, causal=1, scale=0.125, ws=10 * A, ws_bytes=1 << 12):
    return _lib.fa_bwd_raw(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, Tq, Tk, d, causal, scale, ws, ws_bytes, 0)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"])
def test_bwd_null_pointer(lib, which):
    assert bcall(**{which: 0}) == _lib.FA_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), _lib.FA_ERR_SHAPE), (dict(Tq=0), _lib.FA_ERR_SHAPE), (dict(Hq=3, Hkv=2), _lib.FA_ERR_SHAPE),
    (dict(Tq=17, Tk=16), _lib.FA_ERR_SHAPE), (dict(d=96), _lib.FA_ERR_HEAD_DIM),
    (dict(scale=math.nan), _lib.FA_ERR_SCALE), (dict(scale=-3e38), _lib.FA_ERR_SCALE), (dict(causal=2), _lib.FA_ERR_ARG),
    (dict(dq=7 * A + 8), _lib.FA_ERR_ALIGN), (dict(lse=6 * A + 2), _lib.FA_ERR_ALIGN),
    (dict(ws_bytes=16 * 8 - 1), _lib.FA_ERR_ARG), (dict(dk=2 * A), _lib.FA_ERR_ARG),
    (dict(dq=7 * A, dv=7 * A + 16), _lib.FA_ERR_ARG), (dict(ws=A + 64), _lib.FA_ERR_ARG),
    (dict(Tq=1 << 31, Tk=1 << 31), _lib.FA_ERR_OVERFLOW),
])
def test_bwd_rejects(lib, kw, code):
    assert bcall(**kw) == code


def test_bwd_workspace_bytes(lib):
    assert _lib.bwd_workspace_bytes(2, 3, 5) == 2 * 3 * 5 * 8
    assert _lib.bwd_workspace_bytes(0, 3, 5) == 0
    assert lib.fa_hip_error_string() == b""


def test_library_exports_nothing_undeclared(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == _declared_functions(), exported ^ _declared_functions()


def fcall(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, Hq=1, Hkv=1, Tq=16, Tk=16, d=64, causal=1, scale=0.125,
          qd=0.01, kd=0.02, vd=0.03):
    return _lib.fa_fwd_fp8_raw(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, qd, kd, vd, 0)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fp8_null_pointer(lib, which):
    assert fcall(**{which: 0}) == _lib.FA_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), _lib.FA_ERR_SHAPE), (dict(Tk=0), _lib.FA_ERR_SHAPE), (dict(Hq=3, Hkv=2), _lib.FA_ERR_SHAPE),
    (dict(Tq=17, Tk=16), _lib.FA_ERR_SHAPE), (dict(d=96), _lib.FA_ERR_HEAD_DIM), (dict(d=32), _lib.FA_ERR_HEAD_DIM),
    (dict(scale=math.inf), _lib.FA_ERR_SCALE), (dict(qd=0.0), _lib.FA_ERR_SCALE), (dict(kd=-1.0), _lib.FA_ERR_SCALE),
    (dict(vd=math.nan), _lib.FA_ERR_SCALE), (dict(vd=math.inf), _lib.FA_ERR_SCALE),
    (dict(scale=1e30, qd=1e10, kd=1e10), _lib.FA_ERR_SCALE), (dict(causal=3), _lib.FA_ERR_ARG),
    (dict(q=A + 8), _lib.FA_ERR_ALIGN), (dict(o=4 * A + 4), _lib.FA_ERR_ALIGN), (dict(lse=5 * A + 1), _lib.FA_ERR_ALIGN),
    (dict(o=A + 16), _lib.FA_ERR_ARG), (dict(lse=3 * A + 16), _lib.FA_ERR_ARG), (dict(o=4 * A, lse=4 * A + 64), _lib.FA_ERR_ARG),
    (dict(Tq=1 << 31, Tk=1 << 31), _lib.FA_ERR_OVERFLOW), (dict(B=1 << 40, Hq=1 << 30, Hkv=1 << 30), _lib.FA_ERR_OVERFLOW),
])
def test_fp8_rejects(lib, kw, code):
    assert fcall(**kw) == code
    assert lib.fa_hip_error_string() == b""


def test_fp8_python_wrapper_rejects_bf16_and_cpu():
    import torch
    x = torch.zeros((1, 1, 16, 64), dtype=torch.uint8)
    with pytest.raises(ValueError):
        _lib.fwd_fp8(x, x, x, True)                  # CPU tensors
    y = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.fwd_fp8(y, y, y, True)                  # not E4M3 bytes


def scall(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, Hq=1, Hkv=1, Tq=1, Tk=1024, d=128, causal=1, scale=0.125,
          qd=0.01, kd=0.02, vd=0.03, n_split=4, ws=10 * A, ws_bytes=1 << 20):
    return _lib.fa_fwd_fp8_split_raw(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, qd, kd, vd, n_split, ws,
                                     ws_bytes, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(n_split=0), _lib.FA_ERR_ARG), (dict(n_split=-3), _lib.FA_ERR_ARG), (dict(ws=0), _lib.FA_ERR_NULL),
    (dict(ws_bytes=4 * 129 * 4 - 1), _lib.FA_ERR_ARG), (dict(ws=10 * A + 8), _lib.FA_ERR_ALIGN),
    (dict(ws=A), _lib.FA_ERR_ARG), (dict(ws=4 * A), _lib.FA_ERR_ARG), (dict(vd=0.0), _lib.FA_ERR_SCALE),
    (dict(d=96), _lib.FA_ERR_HEAD_DIM), (dict(Tq=2, Tk=1), _lib.FA_ERR_SHAPE), (dict(q=0), _lib.FA_ERR_NULL),
])
def test_fp8_split_rejects(lib, kw, code):
    assert scall(**kw) == code


def test_fp8_split_workspace_matches_the_bf16_split(lib):
    # 4 splits of 1024 keys for one row need 4 * (128 + 1) floats (the size the
    # rejection cases above are measured against)
    assert _lib.split_workspace_bytes(1, 1, 1, 1024, 128, 4) == 4 * 129 * 4


def test_binding_rejects_bad_workspace():
    """A caller workspace is passed as raw bytes: it must be one contiguous tensor on the inputs' device."""
    import torch
    ok = torch.empty(64, dtype=torch.uint8)
    _lib._check_workspace(ok, ok.device)
    with pytest.raises(TypeError):
        _lib._check_workspace(bytearray(64), ok.device)
    with pytest.raises(ValueError):
        _lib._check_workspace(ok, torch.device("cuda", 0))
    with pytest.raises(ValueError):
        _lib._check_workspace(torch.empty(8, 8, dtype=torch.uint8).t(), ok.device)


def test_c_client_is_built_against_the_library():
    """The plain C client links libfa.so (found beside it) and the HIP runtime."""
    from exact_io_aware_13_amd import build as b
    if not os.path.exists(b.C_CLIENT):
        b.build_c_client(force=True)
    out = subprocess.run(["ldd", b.C_CLIENT], capture_output=True, text=True, check=True).stdout
    assert os.path.join(os.path.dirname(b.C_CLIENT), "libfa.so") in out or "libfa.so =>" in out
    assert "libamdhip64" in out
    assert "fa_fwd_split" in open(b.C_CLIENT_SRC).read()
