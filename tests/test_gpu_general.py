"""GPU parity for the general forward: grouped key/value heads (fa_fwd_gqa),
Tq != Tk with the causal rule on the last Tq positions, and split keys with the
log-sum-exp combine (fa_fwd_split), all against the fp64 oracle on the same
bf16 bits.  Tolerances as for the square forward."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_13_amd import workloads as wl

pytestmark = pytest.mark.gpu

O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


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


def run(fa, qb, kb, vb, causal, scale, n_split=1):
    import torch
    o, lse = fa.fwd(to_dev(qb), to_dev(kb), to_dev(vb), causal, float(scale), n_split=n_split)
    torch.cuda.synchronize()
    return (oracle.widen_bf16(o.view(torch.int16).cpu().numpy().view(np.uint16)),
            lse.cpu().numpy().astype(np.float64))


def check(o, o_ref, lse, lse_ref, label):
    max_abs = float(np.abs(o - o_ref).max())
    rel_l2 = float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref))
    lse_abs = float(np.abs(lse - lse_ref).max())
    say(f"[{label}] O max-abs {max_abs:.3e} rel-L2 {rel_l2:.3e} lse max-abs {lse_abs:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), label
    assert max_abs <= O_MAX_ABS and rel_l2 <= O_REL_L2 and lse_abs <= LSE_MAX_ABS, label


def case(fa, B, Hq, Hkv, Tq, Tk, d, causal, n_split=1, seed=0):
    label = f"B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} causal={causal} splits={n_split}"
    say("case", label)
    qb = draw((B, Hq, Tq, d), 100 + seed)
    kb = draw((B, Hkv, Tk, d), 200 + seed)
    vb = draw((B, Hkv, Tk, d), 300 + seed)
    scale = np.float32(1.0 / math.sqrt(d))
    o, lse = run(fa, qb, kb, vb, causal, scale, n_split)
    o_ref, lse_ref = oracle.attention_f64(qb, kb, vb, causal, float(scale))
    check(o, o_ref, lse, lse_ref, label)
    return o, lse


GQA = [(1, 32, 8, 1024, 1024, 128, True), (2, 8, 1, 300, 300, 64, False), (1, 4, 4, 129, 129, 128, True),
       (1, 6, 2, 4097, 4097, 64, True), (1, 8, 2, 8200, 8200, 128, True)]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal", GQA, ids=lambda x: str(x))
def test_grouped_heads(fa, B, Hq, Hkv, Tq, Tk, d, causal):
    case(fa, B, Hq, Hkv, Tq, Tk, d, causal)


RECT = [(1, 4, 2, 100, 1000, 128, True), (1, 4, 2, 100, 1000, 64, False), (2, 2, 2, 700, 130, 64, False),
        (1, 8, 8, 1, 4096, 128, True), (1, 2, 1, 257, 257, 128, True), (1, 2, 1, 63, 64, 64, True)]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal", RECT, ids=lambda x: str(x))
def test_queries_and_keys_differ(fa, B, Hq, Hkv, Tq, Tk, d, causal):
    case(fa, B, Hq, Hkv, Tq, Tk, d, causal)


SPLIT = [(1, 8, 2, 1, 3000, 128, True, 4), (2, 8, 2, 7, 3000, 64, False, 3), (1, 4, 1, 130, 2049, 128, True, 5),
         (1, 4, 4, 1000, 1000, 64, True, 4), (1, 2, 2, 64, 200, 128, False, 16), (1, 2, 1, 3, 70, 64, True, 2),
         (1, 32, 8, 1, 32768, 128, True, None), (4, 32, 8, 1, 4096, 128, False, None),
         # long rows at d = 128 take the 8-wave workgroup with split keys
         (1, 1, 1, 8200, 8200, 128, True, None), (1, 2, 2, 4100, 4100, 128, False, 3)]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,d,causal,n_split", SPLIT, ids=lambda x: str(x))
def test_split_keys(fa, B, Hq, Hkv, Tq, Tk, d, causal, n_split):
    case(fa, B, Hq, Hkv, Tq, Tk, d, causal, n_split)


def test_split_agrees_with_unsplit(fa):
    """The same problem with 1 and with 6 splits: both within tolerance of each other."""
    B, Hq, Hkv, Tq, Tk, d = 1, 4, 2, 200, 5000, 128
    qb, kb, vb = draw((B, Hq, Tq, d), 7), draw((B, Hkv, Tk, d), 8), draw((B, Hkv, Tk, d), 9)
    o1, l1 = run(fa, qb, kb, vb, True, 1.0 / math.sqrt(d), 1)
    o6, l6 = run(fa, qb, kb, vb, True, 1.0 / math.sqrt(d), 6)
    assert np.abs(o1 - o6).max() <= 2 * O_MAX_ABS and np.abs(l1 - l6).max() <= 2 * LSE_MAX_ABS


def test_grouped_equals_replicated(fa):
    """fa_fwd_gqa gives exactly the bits of fa_fwd on key/value heads repeated per group."""
    import torch
    B, Hq, Hkv, T, d = 1, 8, 2, 513, 128
    qb, kb, vb = draw((B, Hq, T, d), 11), draw((B, Hkv, T, d), 12), draw((B, Hkv, T, d), 13)
    g = Hq // Hkv
    og, lg = fa.fwd(to_dev(qb), to_dev(kb), to_dev(vb), True)
    orp, lrp = fa.fwd(to_dev(qb), to_dev(np.repeat(kb, g, axis=1)), to_dev(np.repeat(vb, g, axis=1)), True)
    torch.cuda.synchronize()
    assert torch.equal(og.view(torch.int16), orp.view(torch.int16)) and torch.equal(lg, lrp)


def test_split_workspace_reuse_and_stream(fa):
    """A caller workspace reused over calls of different sizes, on a side stream."""
    import torch
    s = torch.cuda.Stream()
    need = max(fa.split_workspace_bytes(1, 4, 5, 3000, 64, 4), fa.split_workspace_bytes(1, 4, 2, 900, 64, 3))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    for (Tq, Tk, ns, seed) in ((5, 3000, 4, 21), (2, 900, 3, 22)):
        qb, kb, vb = draw((1, 4, Tq, 64), seed), draw((1, 2, Tk, 64), seed + 1), draw((1, 2, Tk, 64), seed + 2)
        q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
        o = torch.empty_like(q)
        lse = torch.empty((1, 4, Tq), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            fa.fwd_out(q, k, v, o, lse, True, 0.125, n_split=ns, workspace=ws)
        s.synchronize()
        o_ref, l_ref = oracle.attention_f64(qb, kb, vb, True, 0.125)
        check(oracle.widen_bf16(o.view(torch.int16).cpu().numpy().view(np.uint16)), o_ref,
              lse.cpu().numpy().astype(np.float64), l_ref, f"reuse Tq={Tq} Tk={Tk}")


def test_workload_gqa_prefill_sampled_rows(fa):
    """Llama-3.1-8B GQA causal prefill at T=8192: seeded sample rows against the oracle."""
    w = wl.BY_KEY["gqa"]
    say("case gqa:", w.title)
    qb, kb, vb = wl.workload_inputs(w)
    scale = np.float32(w.scale)
    o, lse = run(fa, qb, kb, vb, w.causal, scale)
    rows = wl.sample_rows(w)
    o_ref, lse_ref = oracle.attention_rows_f64(qb, kb, vb, w.causal, float(scale), rows)
    check(o.reshape(-1, w.d)[rows], o_ref, lse.reshape(-1)[rows], lse_ref, f"gqa {len(rows)} sampled rows")


def test_workload_decode_every_row(fa):
    """Llama-3.1-8B GQA decode over a 32K-key cache with the library's split count: every row."""
    w = wl.BY_KEY["decode"]
    n_split = fa.split_count(w.B, w.H, w.Hkv, w.T, w.Tk, w.d, w.causal)
    say("case decode:", w.title, "splits", n_split)
    assert n_split > 1
    qb, kb, vb = wl.workload_inputs(w)
    scale = np.float32(w.scale)
    o, lse = run(fa, qb, kb, vb, w.causal, scale, n_split)
    o_ref, lse_ref = oracle.attention_f64(qb, kb, vb, w.causal, float(scale))
    check(o, o_ref, lse, lse_ref, "decode")
