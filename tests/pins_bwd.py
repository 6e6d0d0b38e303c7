"""Pins for the attention backward.

Each pin takes ``grad(q, k, v, do, causal, scale) -> (dq, dk, dv)`` with q, do
of shape (B, Hq, Tq, d) and k, v of shape (B, Hkv, Tk, d), and checks it
against something other than itself.  The gradients are those of
O = softmax(scale * Q K^T [+ causal mask]) V for an upstream gradient dO, the
backward that "FlashAttention and Fused Kernels: Attention Without the n x n
Matrix" ("Training: recompute instead of store") computes by recomputing the
score and probability tiles; the pages state no formulas for it, so the pins
rest on the mathematics:

* torch's float64 CPU autograd through the explicit masked-softmax formula (a
  library differentiation of the forward definition);
* central finite differences of a plain numpy forward along random directions;
* identities that hold for any input: the gradient of the scores sums to zero
  over each row (so dK sums to zero over the keys of a head), every softmax row
  sums to one (so dV summed over keys equals dO summed over rows),
  <dQ, Q> = <dK, K> (both are sum_ij dS_ij s_ij), and <dV, V> = <dO, O>
  (O is linear in V);
* the closed form for equal scores (zero queries), on the worked example of
  "Flash Attention, tiled: exact attention without the T x T HBM matrix"
  ("A three-token example": T = 3, d = 2, zero Q and K), where every
  softmax row is uniform over its visible keys;
* grouped heads equal one head per query head with K, V repeated, the dK, dV
  of a key/value head being the sum over its group;
* with Tq < Tk causal, the rows are the tail of the square problem whose
  earlier rows carry a zero upstream gradient.
"""
import json
import os

import numpy as np

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _fwd(q, k, v, causal, scale):
    """Plain full-matrix forward (numpy, float64), for the finite differences and identities."""
    g = q.shape[1] // k.shape[1]
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    s = scale * np.einsum("bhid,bhjd->bhij", q, kr)
    Tq, Tk = q.shape[2], k.shape[2]
    if causal:
        vis = np.arange(Tk)[None, :] <= np.arange(Tq)[:, None] + (Tk - Tq)
        s = np.where(vis, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("bhij,bhjd->bhid", p, vr)


SHAPES = (  # (B, Hq, Hkv, Tq, Tk, d, causal)
    (1, 1, 1, 6, 6, 4, True),
    (2, 2, 2, 9, 9, 5, False),
    (1, 4, 2, 7, 7, 3, True),
    (2, 3, 1, 5, 11, 4, False),
    (1, 2, 2, 4, 10, 6, True),
    (1, 2, 1, 1, 8, 4, True),
)


def _inputs(rng, B, Hq, Hkv, Tq, Tk, d, s=1.0):
    return (_rand(rng, B, Hq, Tq, d, s=s), _rand(rng, B, Hkv, Tk, d, s=s), _rand(rng, B, Hkv, Tk, d),
            _rand(rng, B, Hq, Tq, d))


def pin_bwd_torch_autograd(grad):
    """torch float64 autograd through softmax(scale Q K^T + mask) V agrees to 1e-12."""
    import torch
    rng = np.random.default_rng(41)
    for (B, Hq, Hkv, Tq, Tk, d, causal) in SHAPES:
        q, k, v, do = _inputs(rng, B, Hq, Hkv, Tq, Tk, d, s=1.2)
        scale = 0.45
        Q, K, V = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
        g = Hq // Hkv
        Kr, Vr = K.repeat_interleave(g, dim=1), V.repeat_interleave(g, dim=1)
        s = scale * Q @ Kr.transpose(-1, -2)
        if causal:
            vis = torch.ones(Tq, Tk, dtype=torch.bool).tril(Tk - Tq)
            s = s.masked_fill(~vis, float("-inf"))
        (torch.softmax(s, dim=-1) @ Vr).backward(torch.from_numpy(do))
        dq, dk, dv = grad(q, k, v, do, causal, scale)
        for got, ref in ((dq, Q.grad), (dk, K.grad), (dv, V.grad)):
            ref = ref.numpy()
            assert got.shape == ref.shape, (got.shape, ref.shape)
            assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), np.abs(got - ref).max()


def pin_bwd_finite_differences(grad):
    """<grad, u> matches the central difference of L = <O, dO> along random directions u."""
    rng = np.random.default_rng(42)
    h = 1e-5
    for (B, Hq, Hkv, Tq, Tk, d, causal) in SHAPES:
        q, k, v, do = _inputs(rng, B, Hq, Hkv, Tq, Tk, d)
        scale = 0.6
        dq, dk, dv = grad(q, k, v, do, causal, scale)

        def loss(q_, k_, v_):
            return float(np.sum(_fwd(q_, k_, v_, causal, scale) * do))

        for which, g in ((0, dq), (1, dk), (2, dv)):
            u = rng.standard_normal(g.shape)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = args_p[which] + h * u
            args_m[which] = args_m[which] - h * u
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            an = float(np.sum(g * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def pin_bwd_identities(grad):
    """sum_j dK_j = 0; sum_j dV_j = sum_i dO_i; <dQ, Q> = <dK, K>; <dV, V> = <dO, O>."""
    rng = np.random.default_rng(43)
    for (B, Hq, Hkv, Tq, Tk, d, causal) in SHAPES:
        q, k, v, do = _inputs(rng, B, Hq, Hkv, Tq, Tk, d, s=1.5)
        scale = 0.7
        dq, dk, dv = grad(q, k, v, do, causal, scale)
        tol = 1e-11
        assert np.abs(dk.sum(axis=2)).max() <= tol * max(1.0, np.abs(dk).max())
        g = Hq // Hkv
        do_sum = do.reshape(B, Hkv, g, Tq, d).sum(axis=(2, 3))
        assert np.abs(dv.sum(axis=2) - do_sum).max() <= tol * max(1.0, np.abs(do_sum).max())
        a, b = float(np.sum(dq * q)), float(np.sum(dk * k))
        assert abs(a - b) <= tol * max(1.0, abs(a)), (a, b)
        o = _fwd(q, k, v, causal, scale)
        a, b = float(np.sum(dv * v)), float(np.sum(do * o))
        assert abs(a - b) <= tol * max(1.0, abs(a)), (a, b)


def pin_bwd_worked_example_uniform(grad):
    """Zero Q and K (T = 3, d = 2, causal; V rows [10, 0], [0, 20], [30, 30]): every row is
    uniform over its visible keys, so dV_j = sum_{i >= j} dO_i / (i + 1) and dQ = dK = 0.
    With zero Q only, dK = 0 and dQ_i = scale * sum_j P_ij (dP_ij - mean_j dP_ij) k_j."""
    with open(os.path.join(_GOLDEN, "w1_three_token_causal.json")) as f:
        ex = json.load(f)
    v = np.array(ex["v"], dtype=np.float64)[None, None]
    assert np.all(np.array(ex["q"]) == 0) and np.all(np.array(ex["k"]) == 0)
    do = np.array([[1.0, -2.0], [0.5, 3.0], [-4.0, 1.5]])[None, None]
    z = np.zeros((1, 1, 3, 2))
    dq, dk, dv = grad(z, z, v, do, True, 0.5)
    want_dv = np.array([do[0, 0, 0] + do[0, 0, 1] / 2 + do[0, 0, 2] / 3,
                        do[0, 0, 1] / 2 + do[0, 0, 2] / 3,
                        do[0, 0, 2] / 3])
    assert np.abs(dv[0, 0] - want_dv).max() <= 1e-12
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    # zero queries, nonzero keys: the scores are still all zero
    k = np.array([[1.0, 2.0], [-3.0, 0.5], [2.0, -1.0]])[None, None]
    scale = 0.5
    dq, dk, dv = grad(z, k, v, do, True, scale)
    assert np.abs(dk).max() <= 1e-12
    assert np.abs(dv[0, 0] - want_dv).max() <= 1e-12
    for i in range(3):
        n = i + 1
        dp = np.array([do[0, 0, i] @ v[0, 0, j] for j in range(n)])
        ds = (dp - dp.mean()) / n
        want = scale * sum(ds[j] * k[0, 0, j] for j in range(n))
        assert np.abs(dq[0, 0, i] - want).max() <= 1e-12, (i, dq[0, 0, i], want)


def pin_bwd_gqa_is_group_sum(grad):
    """Grouped heads: dQ as with K, V repeated per query head; dK, dV the sum over the group."""
    rng = np.random.default_rng(44)
    for (B, Hq, Hkv, T, d) in ((1, 4, 2, 7, 3), (2, 6, 1, 5, 4)):
        q, k, v, do = _inputs(rng, B, Hq, Hkv, T, T, d)
        g = Hq // Hkv
        kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
        for causal in (True, False):
            dq, dk, dv = grad(q, k, v, do, causal, 0.5)
            dq1, dk1, dv1 = grad(q, kr, vr, do, causal, 0.5)
            assert np.abs(dq - dq1).max() <= 1e-12
            assert np.abs(dk - dk1.reshape(B, Hkv, g, T, d).sum(axis=2)).max() <= 1e-12
            assert np.abs(dv - dv1.reshape(B, Hkv, g, T, d).sum(axis=2)).max() <= 1e-12


def pin_bwd_short_queries_are_the_tail(grad):
    """Tq < Tk causal: the square problem with those rows last and dO = 0 on the rows before."""
    rng = np.random.default_rng(45)
    B, H, Tk, d = 1, 2, 9, 4
    for Tq in (1, 4, 9):
        q, k, v, do = _inputs(rng, B, H, H, Tq, Tk, d)
        dq, dk, dv = grad(q, k, v, do, True, 0.5)
        q_full = np.concatenate([_rand(rng, B, H, Tk - Tq, d), q], axis=2)
        do_full = np.concatenate([np.zeros((B, H, Tk - Tq, d)), do], axis=2)
        dqf, dkf, dvf = grad(q_full, k, v, do_full, True, 0.5)
        assert np.abs(dq - dqf[:, :, Tk - Tq:]).max() <= 1e-12
        assert np.abs(dk - dkf).max() <= 1e-12 and np.abs(dv - dvf).max() <= 1e-12


ALL_PINS = [pin_bwd_torch_autograd, pin_bwd_finite_differences, pin_bwd_identities,
            pin_bwd_worked_example_uniform, pin_bwd_gqa_is_group_sum, pin_bwd_short_queries_are_the_tail]
