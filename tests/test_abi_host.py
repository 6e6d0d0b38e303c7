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


def test_status_strings(lib):
    for code in range(0, 9):
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


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf])
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
