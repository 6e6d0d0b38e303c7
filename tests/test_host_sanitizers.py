"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

A copy of libfa.so is built with the host pass instrumented (each sanitizer
flag behind ``-Xarch_host``, so no device code is), and the host-side ABI tests
(argument validation, status strings, overlap and workspace checks, the
allocation-free entry point's checks) run against it in a child process with
the sanitizer runtime preloaded.  Any out-of-bounds access, use after free or
undefined behaviour (signed overflow, invalid enum values, misaligned access,
...) in those paths fails the test."""
import os
import subprocess
import sys

import pytest

from exact_io_aware_13_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    for clang in ("/opt/rocm/llvm/bin/clang", "clang"):
        try:
            out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                                 text=True, timeout=60).stdout.strip()
        except (OSError, subprocess.TimeoutExpired):
            continue
        if out and os.path.isabs(out) and os.path.exists(out):
            return out
    return None


def test_host_abi_paths_are_clean_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime for the ROCm clang")
    lib = tmp_path / "libfa_sanitized.so"
    flags = [f for f in hip_build.compile_flags() if f != "-O3"] + ["-O1", "-g"]
    flags += ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
              "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [hip_build.hipcc()] + flags + ["-shared", "-o", str(lib)] + hip_build.SRCS
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    script = (
        "import sys; sys.path.insert(0, %r)\n"
        "from exact_io_aware_13_amd import _lib\n"
        "_lib.LIB_PATH = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r, '-k', "
        "'not variant and not c_client and not exports']))\n" % (ROOT, str(lib), os.path.join(ROOT, "tests", "test_abi_host.py")))
    # The sanitizer runtime must come first among the preloaded libraries; anything
    # already preloaded in this environment stays, after it.
    preload = ":".join(x for x in (rt, os.environ.get("LD_PRELOAD", "")) if x)
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env, timeout=600)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert " passed" in out
