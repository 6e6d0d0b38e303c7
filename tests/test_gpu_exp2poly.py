"""GPU parity of the polynomial-exponential variant of the forward.

``libfa_exp2poly.so`` is the forward built with 4 of every 32 weights per
lane and key tile taken from the cubic 2^x on the FMA path (FA4's split of the
exponentials between the two units: "FlashAttention and Fused Kernels", "Four
generations of FlashAttention") instead of ``v_exp_f32``.  It is a measurement
variant: ``libfa.so`` takes no polynomial weights at either head size.  Its
results are held to the forward's own bar against the fp64 oracle, and one
closed form checks that masked keys still weigh exactly 0.
"""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_13_amd import workloads as wl

pytestmark = pytest.mark.gpu

O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_io_aware_13_amd as fa
    oracle.build(force=False)
    return fa, fa.load(fa.variant_path("exp2poly"))


def draw(shape, seed, mult=1.0):
    rng = np.random.default_rng(seed)
    return wl.f32_to_bf16_bits(mult * rng.standard_normal(size=shape, dtype=np.float32))


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def run(fa, lib, qb, kb, vb, causal, scale, n_split=1):
    import torch
    o, lse = fa.fwd(to_dev(qb), to_dev(kb), to_dev(vb), causal, float(scale), n_split=n_split, lib=lib)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy().astype(np.float64)


CASES = [
    # B, Hq, Hkv, Tq, Tk, d, causal, n_split, scale (None = 1/sqrt(d))
    (8, 12, 12, 1024, 1024, 64, True, 1, None),      # GPT-2 shape, three 4-wave workgroups per CU
    (2, 4, 4, 1000, 1000, 64, False, 1, None),
    (1, 2, 2, 257, 257, 128, True, 1, None),         # ragged tail
    (1, 4, 4, 8200, 8200, 128, True, 1, None),       # the 8-wave ping-pong kernel
    # scores with a spread of ~4.5 log2 units: rows rescale.  Much larger scales make rows nearly one-hot
    # with |O| >= 4, where rounding O to bf16 alone (half a spacing: 2^-6) exceeds the 1e-2 bar.
    (1, 2, 2, 4100, 4100, 128, False, 1, 0.25),
    (1, 2, 2, 700, 700, 64, True, 1, -0.5),          # negative scale
    (1, 8, 2, 4, 3000, 128, True, 4, None),          # grouped heads, split keys
]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,n_split,scale", CASES, ids=lambda x: str(x))
def test_exp2poly_matches_oracle(env, B, Hq, Hkv, Tq, Tk, d, causal, n_split, scale):
    fa, lib = env
    label = f"exp2poly B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} causal={causal} splits={n_split} scale={scale}"
    say("case", label)
    qb = draw((B, Hq, Tq, d), 11)
    kb = draw((B, Hkv, Tk, d), 12)
    vb = draw((B, Hkv, Tk, d), 13)
    sc = np.float32(1.0 / math.sqrt(d) if scale is None else scale)
    ob, lse = run(fa, lib, qb, kb, vb, causal, sc, n_split)
    o = oracle.widen_bf16(ob)
    o_ref, lse_ref = oracle.attention_f64(qb, kb, vb, causal, float(sc))
    max_abs = float(np.abs(o - o_ref).max())
    rel_l2 = float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref))
    lse_abs = float(np.abs(lse - lse_ref).max())
    say(f"[{label}] O max-abs {max_abs:.3e} rel-L2 {rel_l2:.3e} lse max-abs {lse_abs:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert max_abs <= O_MAX_ABS and rel_l2 <= O_REL_L2 and lse_abs <= LSE_MAX_ABS, label


def test_exp2poly_masked_keys_weigh_zero(env):
    """Causal row 0 sees one key: its one weight is q(0) = 1 exactly and every
    masked weight must be exactly 0, so O_0 is V_0's bits and lse_0 = scale * q_0.k_0
    (up to the polynomial's relative error, which l32 keeps)."""
    fa, lib = env
    B, H, T, d = 2, 4, 300, 64
    qb, kb, vb = draw((B, H, T, d), 21), draw((B, H, T, d), 22), draw((B, H, T, d), 23)
    sc = np.float32(0.125)
    ob, lse = run(fa, lib, qb, kb, vb, True, sc)
    say("exp2poly causal row 0: O_0 == V_0 bit for bit")
    assert np.array_equal(ob[:, :, 0, :], vb[:, :, 0, :])
    s00 = float(sc) * np.einsum("bhd,bhd->bh", oracle.widen_bf16(qb[:, :, 0, :]), oracle.widen_bf16(kb[:, :, 0, :]))
    # l32 is that one weight before its bf16 rounding: within the cubic's 9.5e-5 of 1
    assert np.abs(lse[:, :, 0] - s00).max() <= 2e-4
