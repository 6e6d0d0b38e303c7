"""The seeded input generators (no attention arithmetic in them)."""
import numpy as np
import torch

from exact_io_aware_13_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draws_are_seeded_and_ordered():
    a = wl.draw_bf16((1, 2, 16, 8), seed=3)
    b = wl.draw_bf16((1, 2, 16, 8), seed=3)
    c = wl.draw_bf16((1, 2, 16, 8), seed=4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    q32, k32, v32 = wl.draw_f32((1, 2, 16, 8), seed=3)
    rng = np.random.default_rng(3)
    assert np.array_equal(q32, rng.standard_normal((1, 2, 16, 8), dtype=np.float32))


def test_spikes():
    shape = (1, 2, 4096, 4)
    q, k, v = wl.draw_f32(shape, seed=5, spikes=True)
    q0, k0, v0 = wl.draw_f32(shape, seed=5, spikes=False)
    qm, km = wl.spike_masks(shape, seed=5)
    assert np.array_equal(q[qm], q0[qm] * 8) and np.array_equal(q[~qm], q0[~qm])
    assert np.array_equal(k[km], k0[km] * 8) and np.array_equal(v, v0)
    assert 0.005 < qm.mean() < 0.015 and 0.005 < km.mean() < 0.015


def test_sample_rows():
    w = wl.BY_KEY["c5"]
    small = wl.Workload("t", "t", 1, 8, 1000, 64, True, seed=5, spikes=True)
    qm, _ = wl.spike_masks(small.shape, small.seed)
    rows = wl.sample_rows(small, q_mask=qm)
    assert rows.shape == (256,) and len(set(rows.tolist())) == 256
    heads = sorted(set((rows // small.T).tolist()))
    assert len(heads) == 4
    for h in heads:
        r = rows[rows // small.T == h] % small.T
        assert {0, 1, 63, 64, 127, 128, small.T - 1} <= set(r.tolist())
    assert w.flops() == 4.0 * 32 * 32768 ** 2 * 128 / 2


def test_workload_table():
    c4 = wl.BY_KEY[wl.BENCH_KEY]
    assert (c4.B, c4.H, c4.T, c4.d, c4.causal) == (1, 32, 8192, 128, True)
    assert abs(c4.flops() - 549.755813888e9) < 1e3
    assert c4.algorithmic_bytes() == 8 * 32 * 8192 * 128 + 4 * 32 * 8192


def test_grad_output_draw_is_seeded_and_separate():
    w = wl.BY_KEY["c1"]
    a, b = wl.workload_grad_output(w), wl.workload_grad_output(w)
    assert a.dtype == np.uint16 and a.shape == w.shape and np.array_equal(a, b)
    q, _, _ = wl.workload_inputs(w)
    assert not np.array_equal(a, q)
    x = wl.bf16_bits_to_f32(a)
    assert abs(float(x.mean())) < 0.1 and 0.9 < float(x.std()) < 1.1
