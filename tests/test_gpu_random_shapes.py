"""Seeded random shapes against the fp64 oracle, for the forward (every entry
point the binding picks: fa_fwd, fa_fwd_gqa, fa_fwd_split with given or
advised split counts) and the backward.  The shapes are drawn once from a
fixed seed: batch 1-3, 1-4 key/value heads each shared by 1, 2 or 4 query
heads, query and key lengths from 1 to ~2500 (causal only where Tq <= Tk),
head size 64 or 128, scales within 2/sqrt(d) in magnitude (where no row is so
peaked that |O| reaches 4 and bf16's own spacing exceeds the bar).  Bars as in
the fixed-shape tests: O max-abs 1e-2, rel-L2 5e-3, lse max-abs 1e-3; the
backward's per-gradient rel-L2 1e-2 and max-abs 1e-2 * max(1, max|ref|)."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_13_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _shapes(n, seed, t_max):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 1, 2, 4]))
        d = int(rng.choice([64, 128]))
        Tk = int(rng.choice([int(rng.integers(1, 130)), int(rng.integers(130, t_max))]))
        Tq = Tk if rng.random() < 0.6 else int(rng.integers(1, t_max))
        causal = bool(rng.random() < 0.6) and Tq <= Tk
        scale = float(np.float32(rng.choice([1.0, 0.5, 2.0, -1.0, 0.0]) / math.sqrt(d)))
        n_split = [1, None, int(rng.integers(2, 6))][int(rng.integers(0, 3))]
        out.append((B, Hq, Hkv, Tq, Tk, d, causal, scale, n_split))
    return out


FWD = _shapes(40, 2026, 2600)
BWD = _shapes(14, 7, 900)


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_io_aware_13_amd as fa
    fa.load()
    oracle.build(force=False)
    return fa


def say(*a):
    print(*a, flush=True)


def draw(shape, seed):
    rng = np.random.default_rng(seed)
    return wl.f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def to_f64(t):
    import torch
    return oracle.widen_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("case", range(len(FWD)))
def test_random_forward(fa, case):
    import torch
    B, Hq, Hkv, Tq, Tk, d, causal, scale, n_split = FWD[case]
    label = f"fwd B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} causal={causal} scale={scale:.4g} splits={n_split}"
    say("case", label)
    qb, kb, vb = draw((B, Hq, Tq, d), 3 * case), draw((B, Hkv, Tk, d), 3 * case + 1), draw((B, Hkv, Tk, d), 3 * case + 2)
    o, lse = fa.fwd(to_dev(qb), to_dev(kb), to_dev(vb), causal, scale, n_split=n_split)
    torch.cuda.synchronize()
    o, lse = to_f64(o), lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention_f64(qb, kb, vb, causal, scale)
    max_abs = float(np.abs(o - o_ref).max())
    rel = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-30))
    lerr = float(np.abs(lse - lse_ref).max())
    say(f"[{label}] O max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse max-abs {lerr:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert max_abs <= 1e-2 and rel <= 5e-3 and lerr <= 1e-3, label


@pytest.mark.parametrize("case", range(len(BWD)))
def test_random_backward(fa, case):
    import torch
    B, Hq, Hkv, Tq, Tk, d, causal, scale, _ = BWD[case]
    label = f"bwd B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} causal={causal} scale={scale:.4g}"
    say("case", label)
    qb, kb, vb, dob = (draw((B, Hq, Tq, d), 4 * case + 100), draw((B, Hkv, Tk, d), 4 * case + 101),
                       draw((B, Hkv, Tk, d), 4 * case + 102), draw((B, Hq, Tq, d), 4 * case + 103))
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    o, lse = fa.fwd(q, k, v, causal, scale, n_split=1)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd_f64(qb, kb, vb, dob, causal, scale)
    for name, got, ref in zip(("dq", "dk", "dv"), (to_f64(dq), to_f64(dk), to_f64(dv)), refs):
        R = max(1.0, float(np.abs(ref).max()))
        max_abs = float(np.abs(got - ref).max())
        rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
        say(f"[{label}] {name}: max-abs {max_abs:.3e} (R {R:.2f}) rel-L2 {rel:.3e}")
        assert np.all(np.isfinite(got)), (label, name)
        if np.linalg.norm(ref) == 0.0:
            assert max_abs == 0.0, (label, name)
        else:
            assert max_abs <= 1e-2 * R and rel <= 1e-2, (label, name)
