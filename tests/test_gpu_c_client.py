"""The C ABI from a plain C program (``fa_c_client``, built by
``build.build_c_client`` from ``csrc/fa_c_client.c``): hipMalloc'd buffers,
``fa_fwd``, ``fa_fwd_split`` with a caller workspace, ``fa_bwd``, and two calls
that must be rejected.  Its inputs are a fixed integer hash rounded to bf16,
rebuilt here bit for bit; its outputs are checked against the fp64 oracle with
the bars of the Python-side tests."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from exact_io_aware_13_amd import build as hip_build

pytestmark = pytest.mark.gpu

B, H, T, D = 1, 2, 300, 64
SCALE = 0.125


def input_bits(seed: int, n: int) -> np.ndarray:
    """The client's inputs: value i of stream ``seed`` is an integer hash of i
    mapped to [-2, 2) in fp32, then rounded to bf16 (nearest, ties to even)."""
    i = np.arange(n, dtype=np.uint64)
    x = (i * 2654435761 + seed * 40503 + 12345) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 2246822519) & 0xFFFFFFFF
    x ^= x >> 13
    f = (x >> 8).astype(np.float32) / np.float32(16777216.0) * np.float32(4.0) - np.float32(2.0)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_c_client_matches_the_oracle(tmp_path):
    exe = hip_build.C_CLIENT
    assert os.path.exists(exe), "fa_c_client is not built (run __graft_entry__.build())"
    out = tmp_path / "out.bin"
    print(f"case C client B={B} H={H} T={T} d={D} causal scale={SCALE}", flush=True)
    res = subprocess.run([exe, str(out)], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    n, rows = B * H * T * D, B * H * T
    raw = out.read_bytes()
    assert len(raw) == 2 * (2 * n + 4 * rows) + 3 * 2 * n
    pos = 0

    def take(dtype, count):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=pos)
        pos += a.nbytes
        return a

    o1, l1 = take(np.uint16, n), take(np.float32, rows)
    o2, l2 = take(np.uint16, n), take(np.float32, rows)
    dq, dk, dv = take(np.uint16, n), take(np.uint16, n), take(np.uint16, n)
    shape = (B, H, T, D)
    qb, kb, vb, dob = (input_bits(s, n).reshape(shape) for s in (1, 2, 3, 4))
    o_ref, lse_ref = oracle.attention_f64(qb, kb, vb, True, SCALE)
    for name, o, l in (("fa_fwd", o1, l1), ("fa_fwd_split", o2, l2)):
        o64 = oracle.widen_bf16(o.reshape(shape))
        max_abs = float(np.abs(o64 - o_ref).max())
        rel = float(np.linalg.norm(o64 - o_ref) / np.linalg.norm(o_ref))
        lerr = float(np.abs(l.reshape(B, H, T).astype(np.float64) - lse_ref).max())
        print(f"[{name}] O max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse max-abs {lerr:.3e}", flush=True)
        assert max_abs <= 1e-2 and rel <= 5e-3 and lerr <= 1e-3, name
    refs = oracle.attention_bwd_f64(qb, kb, vb, dob, True, SCALE)
    for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g64 = oracle.widen_bf16(g.reshape(shape))
        R = max(1.0, float(np.abs(ref).max()))
        max_abs = float(np.abs(g64 - ref).max())
        rel = float(np.linalg.norm(g64 - ref) / np.linalg.norm(ref))
        print(f"[fa_bwd {name}] max-abs {max_abs:.3e} (R {R:.2f}) rel-L2 {rel:.3e}", flush=True)
        assert max_abs <= 1e-2 * R and rel <= 1e-2, name
