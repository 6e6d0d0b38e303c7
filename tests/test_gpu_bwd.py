"""GPU parity for the backward (fa_bwd) against the fp64 oracle on the same bf16 bits.

The GPU backward takes O and lse from the GPU forward (what training does);
the oracle computes the exact gradients of the same bf16-rounded q, k, v for
the same upstream gradient dO.  One case also feeds the oracle's own O and lse
to the GPU backward, to separate the backward's error from the forward's.

Tolerance (per gradient, relative to its largest entry R = max(1, max|ref|)):
rel-L2 <= 1e-2 and max-abs <= 1e-2 * R.  The derivation: the outputs are
rounded to bf16 (relative error <= 2^-9, rms 2^-9 / sqrt(3) ~ 1.1e-3), and the
two products that feed them use bf16 roundings of P and dS as operands (each
<= 2^-9 relative, summed with random signs), so the expected rel-L2 is about
2e-3 and the largest elementwise error a few 2^-9 of the largest entry; the
bounds leave a factor of 4-5 above that.
"""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_13_amd import workloads as wl

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS_REL = 1e-2


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


def draw(shape, seed, s=1.0):
    rng = np.random.default_rng(seed)
    return wl.f32_to_bf16_bits((rng.standard_normal(size=shape, dtype=np.float32) * np.float32(s)))


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def to_f64(t):
    import torch
    return oracle.widen_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))


def check(name, got, ref, label):
    R = max(1.0, float(np.abs(ref).max()))
    max_abs = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"[{label}] {name}: max-abs {max_abs:.3e} (R {R:.2f}) rel-L2 {rel:.3e}")
    assert np.all(np.isfinite(got)), (label, name)
    assert max_abs <= MAX_ABS_REL * R and rel <= REL_L2, (label, name, max_abs, rel)


def gpu_grads(fa, qb, kb, vb, dob, causal, scale, o=None, lse=None):
    import torch
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    if o is None:
        o, lse = fa.fwd(q, k, v, causal, float(scale), n_split=1)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal, float(scale))
    torch.cuda.synchronize()
    return to_f64(dq), to_f64(dk), to_f64(dv)


def inputs(B, Hq, Hkv, Tq, Tk, d, seed):
    return (draw((B, Hq, Tq, d), 500 + seed), draw((B, Hkv, Tk, d), 600 + seed), draw((B, Hkv, Tk, d), 700 + seed),
            draw((B, Hq, Tq, d), 800 + seed))


CASES = [  # (B, Hq, Hkv, Tq, Tk, d, causal)
    (1, 1, 1, 128, 128, 64, True),
    (1, 1, 1, 128, 128, 64, False),
    (2, 3, 3, 200, 200, 64, False),
    (1, 2, 2, 333, 333, 128, True),
    (1, 4, 2, 256, 256, 128, True),
    (1, 4, 1, 130, 300, 64, True),
    (2, 2, 2, 100, 260, 128, False),
    (1, 2, 2, 600, 130, 128, False),
    (1, 1, 1, 1, 1, 64, True),
    (1, 2, 2, 1, 517, 128, True),
    (1, 1, 1, 64, 64, 128, False),
    (1, 2, 2, 1030, 1030, 64, True),
    (2, 4, 4, 515, 515, 128, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal", CASES, ids=lambda x: str(x))
def test_bwd_parity(fa, B, Hq, Hkv, Tq, Tk, d, causal):
    label = f"bwd B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} causal={causal}"
    say("case", label)
    qb, kb, vb, dob = inputs(B, Hq, Hkv, Tq, Tk, d, seed=Tq + Tk + d)
    scale = np.float32(1.0 / math.sqrt(d))
    dq, dk, dv = gpu_grads(fa, qb, kb, vb, dob, causal, scale)
    rq, rk, rv = oracle.attention_bwd_f64(qb, kb, vb, dob, causal, float(scale))
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(name, got, ref, label)


def test_bwd_with_oracle_forward(fa):
    """The oracle's O (rounded to bf16) and lse as the backward's inputs."""
    import torch
    B, H, T, d = 1, 2, 300, 128
    qb, kb, vb, dob = inputs(B, H, H, T, T, d, seed=11)
    scale = np.float32(1.0 / math.sqrt(d))
    o_ref, lse_ref = oracle.attention_f64(qb, kb, vb, True, float(scale))
    o = to_dev(wl.f32_to_bf16_bits(o_ref.astype(np.float32)))
    lse = torch.from_numpy(lse_ref.astype(np.float32)).to("cuda:0")
    dq, dk, dv = gpu_grads(fa, qb, kb, vb, dob, True, scale, o=o, lse=lse)
    rq, rk, rv = oracle.attention_bwd_f64(qb, kb, vb, dob, True, float(scale))
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(name, got, ref, "oracle O/lse")


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.9])
def test_bwd_scales(fa, scale):
    """Zero (uniform rows), negative and large scales."""
    B, H, T, d = 1, 2, 200, 64
    qb, kb, vb, dob = inputs(B, H, H, T, T, d, seed=int(scale * 10) + 20)
    s = np.float32(scale)
    dq, dk, dv = gpu_grads(fa, qb, kb, vb, dob, True, s)
    rq, rk, rv = oracle.attention_bwd_f64(qb, kb, vb, dob, True, float(s))
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(name, got, ref, f"scale {scale}")


def test_bwd_is_deterministic(fa):
    """No atomics: two calls give the same bits."""
    import torch
    B, Hq, Hkv, T, d = 1, 4, 2, 777, 128
    qb, kb, vb, dob = inputs(B, Hq, Hkv, T, T, d, seed=3)
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    o, lse = fa.fwd(q, k, v, True)
    a = fa.bwd(q, k, v, o, lse, do, True)
    b = fa.bwd(q, k, v, o, lse, do, True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_workspace_and_stream(fa):
    """A caller workspace on a side stream gives the same bits as the default call."""
    import torch
    B, H, T, d = 2, 2, 260, 64
    qb, kb, vb, dob = inputs(B, H, H, T, T, d, seed=4)
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    o, lse = fa.fwd(q, k, v, False)
    ref = fa.bwd(q, k, v, o, lse, do, False)
    torch.cuda.synchronize()
    ws = torch.full((fa.bwd_workspace_bytes(B, H, T) + 64,), 0x7F, dtype=torch.uint8, device="cuda:0")
    outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.bwd_out(q, k, v, o, lse, do, *outs, False, None, workspace=ws)
    side.synchronize()
    for x, y in zip(ref, outs):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


SAMPLED = [  # full-size problems, checked on sampled rows: (B, Hq, Hkv, T, d, causal, heads sampled)
    (1, 32, 32, 8192, 128, True, (0, 31)),
    (1, 32, 8, 4096, 128, True, (5,)),
    (8, 12, 12, 1024, 64, True, (13, 95)),
    (16, 16, 16, 1024, 64, False, (7,)),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,d,causal,heads", SAMPLED, ids=lambda x: str(x))
def test_bwd_full_size_sampled(fa, B, Hq, Hkv, T, d, causal, heads):
    """Full-size shapes: dq rows and dk / dv rows sampled across the sequence of a few heads."""
    label = f"bwd sampled B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} causal={causal}"
    say("case", label)
    qb, kb, vb, dob = inputs(B, Hq, Hkv, T, T, d, seed=T + d + Hkv)
    scale = np.float32(1.0 / math.sqrt(d))
    dq, dk, dv = gpu_grads(fa, qb, kb, vb, dob, causal, scale)
    rng = np.random.default_rng(T)
    qrows, krows = [], []
    for bh in heads:
        b, h = bh // Hq, bh % Hq
        pos = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, 24, replace=False)]))
        qrows += list(bh * T + pos)
        bkv = b * Hkv + h // (Hq // Hkv)
        krows += list(bkv * T + pos)
    krows = sorted(set(krows))
    rq, rk, rv = oracle.attention_bwd_rows_f64(qb, kb, vb, dob, causal, float(scale), qrows, krows)
    d_ = dq.shape[-1]
    check("dq", dq.reshape(-1, d_)[qrows], rq, label)
    check("dk", dk.reshape(-1, d_)[krows], rk, label)
    check("dv", dv.reshape(-1, d_)[krows], rv, label)


def test_bwd_long_context_spiky_sampled(fa):
    """The long-context spiky workload (B=1 H=32 T=32768 d=128, 1% of Q and K rows x8): dq rows
    and dk / dv rows of one head, including spiked query rows and the first and last positions.

    Spiked rows give nearly one-hot softmax rows, where dP - D cancels and the
    bf16 rounding of O in D = dO . O (the only O the backward receives)
    dominates dS.  The bound therefore adds twice that rounding's own effect,
    computed by the oracle alone: the gradients with D_i = dO_i . bf16(O_i),
    O from the oracle forward, against the exact ones."""
    w = wl.BY_KEY["c5"]
    label = "bwd sampled " + w.title
    say("case", label)
    qb, kb, vb = wl.workload_inputs(w)
    dob = wl.workload_grad_output(w)
    scale = np.float32(w.scale)
    dq, dk, dv = gpu_grads(fa, qb, kb, vb, dob, True, scale)
    q_mask, k_mask = wl.spike_masks(w.shape, w.seed)
    h = 17
    rng = np.random.default_rng(5)
    pos = set(int(x) for x in rng.choice(w.T, 20, replace=False)) | {0, 1, 63, 64, w.T - 1}
    pos |= set(int(x) for x in np.flatnonzero(q_mask[0, h])[:6]) | set(int(x) for x in np.flatnonzero(k_mask[0, h])[:6])
    rows = sorted(h * w.T + p for p in pos)
    ref = oracle.attention_bwd_rows_f64(qb, kb, vb, dob, True, float(scale), rows, rows)
    # D from the bf16-rounded oracle O of head h (every row of the head: dK, dV rows need them all)
    head_rows = np.arange(h * w.T, (h + 1) * w.T)
    o_h, _ = oracle.attention_rows_f64(qb, kb, vb, True, float(scale), head_rows)
    o_h16 = oracle.widen_bf16(wl.f32_to_bf16_bits(o_h.astype(np.float32)))
    d_rows = np.zeros((w.B, w.H, w.T))
    d_rows[0, h] = np.einsum("id,id->i", oracle.widen_bf16(dob[0, h]), o_h16)
    ref_d = oracle.attention_bwd_rows_f64(qb, kb, vb, dob, True, float(scale), rows, rows, d_rows=d_rows)
    d_ = w.d
    for name, got, r, rd in (("dq", dq.reshape(-1, d_)[rows], ref[0], ref_d[0]),
                             ("dk", dk.reshape(-1, d_)[rows], ref[1], ref_d[1]),
                             ("dv", dv.reshape(-1, d_)[rows], ref[2], ref_d[2])):
        R = max(1.0, float(np.abs(r).max()))
        e_max = float(np.abs(rd - r).max())
        e_rel = float(np.linalg.norm(rd - r) / max(np.linalg.norm(r), 1e-30))
        max_abs = float(np.abs(got - r).max())
        rel = float(np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30))
        say(f"[{label}] {name}: max-abs {max_abs:.3e} (R {R:.2f}) rel-L2 {rel:.3e}; "
            f"bf16-O-in-D effect max-abs {e_max:.3e} rel-L2 {e_rel:.3e}")
        assert np.all(np.isfinite(got)), name
        assert max_abs <= MAX_ABS_REL * R + 2 * e_max and rel <= REL_L2 + 2 * e_rel, (name, max_abs, rel)
