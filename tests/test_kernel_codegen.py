"""The generated gfx950 code of every forward kernel, checked on the host.

hipcc cross-compiles the device code to assembly (no GPU needed), and the
checks guard properties that decide the kernel's speed but no numerics test
sees:
  * no register spills (scratch traffic in the inner loop);
  * no wait on the tile loads (vmcnt) right before an LDS read: the tile loads
    write LDS directly, and a read of one tile must not wait for the load of
    the next, which would put the HBM latency back on every tile.
"""
import os
import re
import subprocess

import pytest

from exact_io_aware_13_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "fa_fwd.s"
    cmd = [build.hipcc()] + [f for f in build.compile_flags() if f != "-fPIC"] + \
        ["--cuda-device-only", "-S", "-o", str(out), build.SRCS[0]]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _kernels(asm):
    for m in re.finditer(r"^(_ZN\S*fa_fwd_kernel\S*):", asm, re.M):
        start = m.end()
        end = asm.index(".Lfunc_end", start)
        body = [l.strip() for l in asm[start:end].splitlines()]
        yield m.group(1), [l for l in body if l and not l.startswith((";", "."))]


def test_every_variant_is_compiled(asm):
    names = [n for n, _ in _kernels(asm)]
    assert len(names) == 16, names      # d x causal x wave groups x split


def test_no_register_spills(asm):
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm)]
    sgpr_spills = [int(x) for x in re.findall(r"\.sgpr_spill_count:\s+(\d+)", asm)]
    assert spills and max(spills) == 0 and max(sgpr_spills) == 0


@pytest.mark.parametrize("name", sorted(build.VARIANTS))
def test_measurement_variants_compile_every_kernel_without_spills(name, tmp_path):
    out = tmp_path / f"fa_fwd_{name}.s"
    cmd = [build.hipcc()] + [f for f in build.compile_flags() if f != "-fPIC"] + build.VARIANTS[name] + \
        ["--cuda-device-only", "-S", "-o", str(out), build.SRCS[0]]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    assert len(list(_kernels(text))) == 16
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)]
    assert spills and max(spills) == 0
    if name == "exp2poly":      # the polynomial's scaling step is there, and so is v_exp_f32
        assert "v_ldexp_f32" in text and "v_exp_f32" in text


def test_lds_reads_do_not_wait_on_tile_loads(asm):
    for name, body in _kernels(asm):
        waits = [i for i, (a, b) in enumerate(zip(body, body[1:]))
                 if a.startswith("s_waitcnt") and "vmcnt" in a and b.startswith("ds_read")]
        assert not waits, (name, [body[i:i + 2] for i in waits[:3]])


@pytest.fixture(scope="module")
def asm_bwd(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "fa_bwd.s"
    cmd = [build.hipcc()] + [f for f in build.compile_flags() if f != "-fPIC"] + \
        ["--cuda-device-only", "-S", "-o", str(out), build.SRCS[1]]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _bwd_kernels(asm):
    for m in re.finditer(r"^(_ZN\S*fa_bwd_\w+_kernel\S*):", asm, re.M):
        start = m.end()
        end = asm.index(".Lfunc_end", start)
        body = [l.strip() for l in asm[start:end].splitlines()]
        yield m.group(1), [l for l in body if l and not l.startswith((";", "."))]


def test_every_backward_variant_is_compiled(asm_bwd):
    names = [n for n, _ in _bwd_kernels(asm_bwd)]
    assert sum("prep" in n for n in names) == 2, names      # d
    assert sum("dkdv" in n for n in names) == 4, names      # d x causal
    assert sum("dq_kernel" in n for n in names) == 4, names


def test_backward_has_no_register_spills_and_fits_two_waves_per_simd(asm_bwd):
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm_bwd)]
    assert spills and max(spills) == 0
    counts = [int(x) for x in re.findall(r"\.vgpr_count:\s+(\d+)", asm_bwd)]
    assert max(counts) <= 256, counts


def test_backward_lds_reads_do_not_wait_on_tile_loads(asm_bwd):
    for name, body in _bwd_kernels(asm_bwd):
        waits = [i for i, (a, b) in enumerate(zip(body, body[1:]))
                 if a.startswith("s_waitcnt") and "vmcnt" in a and "lgkmcnt" not in a and b.startswith("ds_read")]
        assert not waits, (name, [body[i:i + 2] for i in waits[:3]])


@pytest.fixture(scope="module")
def asm_fp8(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "fa_fwd_fp8.s"
    cmd = [build.hipcc()] + [f for f in build.compile_flags() if f != "-fPIC"] + \
        ["--cuda-device-only", "-S", "-o", str(out), build.SRCS[2]]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _fp8_kernels(asm):
    for m in re.finditer(r"^(_ZN\S*fa_fwd_fp8_kernel\S*):", asm, re.M):
        start = m.end()
        end = asm.index(".Lfunc_end", start)
        body = [l.strip() for l in asm[start:end].splitlines()]
        yield m.group(1), [l for l in body if l and not l.startswith((";", "."))]


def test_fp8_variants_use_the_fp8_matrix_cores(asm_fp8):
    kernels = dict(_fp8_kernels(asm_fp8))
    assert len(kernels) == 12, list(kernels)   # ((d=128 x causal x wave groups) + (d=64 x causal)) x split
    for name, body in kernels.items():
        ops = [l.split()[0] for l in body]
        assert "v_mfma_f32_32x32x64_f8f6f4" in ops, name
        assert "ds_read_b64_tr_b8" in ops and "v_cvt_pk_fp8_f32" in ops, name
        assert not any(o.startswith("v_mfma") and "f8f6f4" not in o for o in ops), name


def test_fp8_no_register_spills_and_two_waves_per_simd(asm_fp8):
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm_fp8)]
    assert spills and max(spills) == 0
    counts = [int(x) for x in re.findall(r"\.vgpr_count:\s+(\d+)", asm_fp8)]
    assert max(counts) <= 256, counts


def test_fp8_lds_reads_do_not_wait_on_tile_loads(asm_fp8):
    for name, body in _fp8_kernels(asm_fp8):
        waits = [i for i, (a, b) in enumerate(zip(body, body[1:]))
                 if a.startswith("s_waitcnt") and "vmcnt" in a and "lgkmcnt" not in a and b.startswith("ds_read")]
        assert not waits, (name, [body[i:i + 2] for i in waits[:3]])

