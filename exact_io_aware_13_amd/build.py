"""Build the gfx950 HIP library ``libfa.so`` in-tree with hipcc.

The library (the bf16 forward, the backward and the FP8 forward) exports the C ABI declared in
``include/fa.h``.  Flags: gfx950
only, -O3, packed-fp32 instructions disabled in the device pass
(``-Xclang -target-feature -Xclang -packed-fp32-ops``; the host pass prints a
harmless notice that it does not know that feature), and ``-fno-honor-nans``:
inputs must be finite, so max reductions need no NaN canonicalisation.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "fa_fwd.hip"), os.path.join(PKG, "csrc", "fa_bwd.hip"),
        os.path.join(PKG, "csrc", "fa_fwd_fp8.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"
# Measurement variants: the same sources built with one compile-time choice
# changed, each a library of its own with the same C ABI.  ``exp2poly`` takes
# 4 of every 32 forward weights from the polynomial 2^x (``kPolyExp2`` in
# fa_fwd.hip) at both head sizes.
VARIANTS = {"exp2poly": ["-DFA_EXP2_POLY=4"]}


def variant_path(name: str) -> str:
    return os.path.join(PKG, f"libfa_{name}.so")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-honor-nans",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in VGPRs: the score tiles feed VALU work directly
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE]


def build(force: bool = True, extra=None, out: str | None = None, quiet: bool = True) -> str:
    """Compile the ``csrc/*.hip`` sources of ``SRCS`` into ``libfa.so``; returns the library path."""
    out = out or LIB
    newest = max(os.path.getmtime(p) for p in SRCS + [os.path.join(INCLUDE, "fa.h"),
                                                      os.path.join(PKG, "csrc", "fa_internal.h")])
    if not force and os.path.exists(out) and os.path.getmtime(out) >= newest:
        return out
    cmd = [hipcc()] + compile_flags() + list(extra or []) + ["-shared", "-o", out + ".tmp"] + SRCS
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msg}")
    if msg.strip() and not quiet:
        print(msg, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


C_CLIENT_SRC = os.path.join(PKG, "csrc", "fa_c_client.c")
C_CLIENT = os.path.join(PKG, "fa_c_client")


def build_c_client(force: bool = True) -> str:
    """Compile ``fa_c_client``, a plain C program that calls ``libfa.so`` through
    ``include/fa.h`` (gcc, linked against the library beside it)."""
    if not force and os.path.exists(C_CLIENT) and os.path.getmtime(C_CLIENT) >= max(
            os.path.getmtime(C_CLIENT_SRC), os.path.getmtime(LIB)):
        return C_CLIENT
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), C_CLIENT_SRC, "-L", PKG, "-lfa", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", C_CLIENT + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(C_CLIENT + ".tmp", C_CLIENT)
    return C_CLIENT


def build_all(force: bool = True, quiet: bool = True) -> list:
    """Build ``libfa.so``, every measurement variant and the C client; returns their paths."""
    out = [build(force=force, quiet=quiet)]
    for name, flags in VARIANTS.items():
        out.append(build(force=force, extra=flags, out=variant_path(name), quiet=quiet))
    out.append(build_c_client(force=force))
    return out


if __name__ == "__main__":
    for path in build_all(force=True, quiet=False):
        print(path)
