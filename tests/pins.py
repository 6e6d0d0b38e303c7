"""Pins: checks that fix what an exact attention forward must return.

Every pin takes an attention callable ``attn(q, k, v, causal, scale) -> (o, lse)``
over float64 arrays of shape (B, H, T, d) and raises AssertionError when the
callable disagrees with something the pages print or the mathematics fixes:

* worked examples printed on the pages (fixtures under ``tests/golden/``);
* closed forms (zero scores give running means; all-ones values give ones;
  row 0 of a causal head sees only key 0);
* invariants (a common shift of every score in a row leaves O alone and moves
  lse by the shift; O is linear in V; keys may be permuted when nothing is
  masked; large scores must not overflow);
* library routines that compute the same function (torch's CPU
  ``scaled_dot_product_attention`` in float64, ``scipy.special.logsumexp``);
* brute force on tiny inputs (the full score and probability matrices).

The same pins run against the CPU oracle (which must pass all of them) and
against deliberately wrong variants (each must fail at least one), see
``test_oracle_pins.py`` and ``test_pins_catch_mutants.py``.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bhtd(x) -> np.ndarray:
    """(T, d) -> (1, 1, T, d) float64."""
    return np.asarray(x, dtype=np.float64)[None, None]


def _printed(value, printed, decimals):
    """|value - printed| must be within the rounding of a number printed with ``decimals``."""
    tol = 0.5 * 10.0 ** (-decimals) + 1e-12
    assert np.all(np.abs(np.asarray(value) - np.asarray(printed)) <= tol), (value, printed)


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------

def pin_w1_three_token(attn):
    """joelfernandes.org, 'A three-token example': outputs, probability rows, and lse."""
    g = golden("w1_three_token_causal.json")
    q, k, v = _bhtd(g["q"]), _bhtd(g["k"]), _bhtd(g["v"])
    scale = 1.0 / math.sqrt(g["d"])
    o, lse = attn(q, k, v, True, scale)
    _printed(o[0, 0], g["Y"], g["Y_printed_decimals"])
    # The exact values the printed ones round: V0, (V0+V1)/2, (V0+V1+V2)/3.
    assert np.allclose(o[0, 0], [[10, 0], [5, 10], [40 / 3, 50 / 3]], rtol=0, atol=1e-12)
    # All visible scores are 0, so lse_i = ln(number of visible keys).
    assert np.allclose(lse[0, 0], [0.0, math.log(2), math.log(3)], rtol=0, atol=1e-12)
    # With V = identity the output rows are the probability rows the page prints.
    z = np.zeros((1, 1, 3, 3))
    p, _ = attn(z, z, _bhtd(np.eye(3)), True, 1.0)
    assert np.allclose(p[0, 0], g["probabilities"], rtol=0, atol=1e-12)


def pin_w2_four_scores(attn):
    """vidyal.ai Step 2 worked example and Step 4 block statistics."""
    g = golden("w2_four_scores.json")
    s = np.asarray(g["scores"])
    vals = np.asarray(g["values"])
    T = len(s)
    # Embed: q = e0, k_j = s_j e0, scale 1, so the scores are exactly s.
    d = 4
    q = np.zeros((T, d)); q[:, 0] = 1.0
    k = np.zeros((T, d)); k[:, 0] = s
    v = np.zeros((T, d)); v[:, 0] = vals
    o, lse = attn(_bhtd(q), _bhtd(k), _bhtd(v), False, 1.0)
    _printed(o[0, 0, :, 0], [g["output"]] * T, g["output_printed_decimals"])
    # The combine's printed denominator 1.553 is sum_j exp(s_j - 4).
    l = math.exp(lse[0, 0, 0] - max(s))
    _printed(l, g["combine"]["denominator"], 3)
    # Weights: V = identity makes the output the weight vector.
    w, _ = attn(_bhtd(q), _bhtd(k), _bhtd(np.eye(T)), False, 1.0)
    _printed(w[0, 0, 0], g["weights"], g["weights_printed_decimals"])
    # Causal: the last row sees every key; row 0 sees key 0 only.
    oc, lc = attn(_bhtd(q), _bhtd(k), _bhtd(v), True, 1.0)
    _printed(oc[0, 0, T - 1, 0], g["output"], g["output_printed_decimals"])
    assert abs(oc[0, 0, 0, 0] - vals[0]) <= 1e-12 and abs(lc[0, 0, 0] - s[0]) <= 1e-12
    # Each block alone (Step 4): max, sum and partial output as printed.
    for blk, sl in (("block1", slice(0, 2)), ("block2", slice(2, 4))):
        ob, lb = attn(_bhtd(q[sl]), _bhtd(k[sl]), _bhtd(v[sl]), False, 1.0)
        st = g[blk]
        _printed(ob[0, 0, 0, 0], st["output"], 2)
        _printed(math.exp(lb[0, 0, 0] - st["max"]), st["sum"], 3)


def pin_w4_online_code(attn):
    """inference-learning-path section 4: the printed 6-decimal output."""
    g = golden("w4_online_softmax_code.json")
    K = np.asarray(g["K"]); V = np.asarray(g["V"])
    T = K.shape[0]
    q = np.tile(np.asarray(g["q"]), (T, 1))
    o, _ = attn(_bhtd(q), _bhtd(K), _bhtd(V), False, g["scale"])
    for i in range(T):
        _printed(o[0, 0, i], g["output"], g["output_printed_decimals"])


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def pin_zero_scores_running_mean(attn, B=2, H=3, T=37, d=8, seed=11):
    """Q = 0: every visible weight is equal, so O_i is the mean of the visible V rows."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, H, T, d)); v = rng.standard_normal((B, H, T, d))
    q = np.zeros((B, H, T, d))
    o, lse = attn(q, k, v, True, 0.7)
    n = np.arange(1, T + 1, dtype=np.float64)
    assert np.allclose(o, np.cumsum(v, axis=2) / n[:, None], rtol=0, atol=1e-12)
    assert np.allclose(lse, np.broadcast_to(np.log(n), (B, H, T)), rtol=0, atol=1e-12)
    o, lse = attn(q, k, v, False, 0.7)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(T), rtol=0, atol=1e-12)


def pin_ones_values(attn, B=1, H=2, T=29, d=16, seed=12):
    """V = 1: probability rows sum to one, so O = 1 whatever the scores."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d)) * 2; k = rng.standard_normal((B, H, T, d)) * 2
    for causal in (True, False):
        o, _ = attn(q, k, np.ones((B, H, T, d)), causal, 0.5)
        assert np.allclose(o, 1.0, rtol=0, atol=1e-12)


def pin_causal_first_row(attn, B=2, H=2, T=19, d=8, seed=13):
    """Causal row 0 sees key 0 only: O_0 = V_0 and lse_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    o, lse = attn(q, k, v, True, 0.3)
    assert np.allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-12)
    assert np.allclose(lse[:, :, 0], 0.3 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), rtol=0, atol=1e-12)


def pin_identity_values_lower_triangular(attn, T=12, d=12, seed=14):
    """V = I (T <= d): O is the probability matrix; causal rows are lower-triangular and sum to 1."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, T, d)); k = rng.standard_normal((1, 1, T, d))
    p, _ = attn(q, k, np.eye(T, d)[None, None], True, 1.0 / math.sqrt(d))
    p = p[0, 0, :, :T]
    assert np.all(np.triu(p, 1) == 0.0)
    assert np.all(p[np.tril_indices(T)] > 0.0)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def pin_shift_invariance(attn, B=1, H=2, T=23, d=8, seed=15):
    """k_j -> k_j + u for every j shifts row i's scores by scale*q_i.u: O fixed, lse moves by it."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    u = rng.standard_normal(d) * 3
    scale = 0.4
    for causal in (True, False):
        o1, l1 = attn(q, k, v, causal, scale)
        o2, l2 = attn(q, k + u, v, causal, scale)
        assert np.allclose(o1, o2, rtol=0, atol=1e-10)
        assert np.allclose(l2 - l1, scale * (q @ u), rtol=0, atol=1e-10)


def pin_linear_in_values(attn, B=1, H=1, T=17, d=8, seed=16):
    """O is linear in V (the weights do not depend on V)."""
    rng = np.random.default_rng(seed)
    q, k, v1, v2 = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    for causal in (True, False):
        oa, la = attn(q, k, v1, causal, 0.5)
        ob, lb = attn(q, k, v2, causal, 0.5)
        oc, lc = attn(q, k, 2.0 * v1 - 3.0 * v2, causal, 0.5)
        assert np.allclose(oc, 2.0 * oa - 3.0 * ob, rtol=0, atol=1e-10)
        assert np.allclose(la, lb, rtol=0, atol=1e-12) and np.allclose(la, lc, rtol=0, atol=1e-12)


def pin_key_permutation(attn, B=1, H=2, T=21, d=8, seed=17):
    """Without a mask, permuting (k_j, v_j) pairs together changes nothing."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    perm = rng.permutation(T)
    o1, l1 = attn(q, k, v, False, 0.5)
    o2, l2 = attn(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def pin_large_scores_no_overflow(attn, T=9, d=4):
    """Scores near 800 overflow exp() unless the row maximum is subtracted first."""
    rng = np.random.default_rng(18)
    q = np.zeros((1, 1, T, d)); q[..., 0] = 1.0
    k = np.zeros((1, 1, T, d)); k[..., 0] = 800.0 + rng.standard_normal(T)
    v = rng.standard_normal((1, 1, T, d))
    k0 = k.copy(); k0[..., 0] -= 800.0
    for causal in (True, False):
        o, lse = attn(q, k, v, causal, 1.0)
        o0, lse0 = attn(q, k0, v, causal, 1.0)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        assert np.allclose(o, o0, rtol=0, atol=1e-10)
        assert np.allclose(lse - 800.0, lse0, rtol=0, atol=1e-10)


# --------------------------------------------------------------------------
# Library routines and brute force
# --------------------------------------------------------------------------

def _random_cases():
    rng = np.random.default_rng(19)
    for T, d in ((1, 1), (2, 3), (5, 2), (16, 4), (33, 64), (64, 8)):
        for causal in (True, False):
            B, H = 2, 2
            q, k, v = (rng.standard_normal((B, H, T, d)) * 1.5 for _ in range(3))
            yield q, k, v, causal, float(rng.uniform(0.1, 1.2))


def pin_torch_sdpa(attn):
    """torch's CPU scaled_dot_product_attention in float64 computes the same O."""
    import torch
    import torch.nn.functional as F
    for q, k, v, causal, scale in _random_cases():
        o, _ = attn(q, k, v, causal, scale)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             is_causal=causal, scale=scale).numpy()
        assert np.allclose(o, ref, rtol=0, atol=1e-12), np.abs(o - ref).max()


def pin_scipy_logsumexp(attn):
    """lse_i equals scipy.special.logsumexp over row i's visible scores."""
    from scipy.special import logsumexp
    for q, k, v, causal, scale in _random_cases():
        _, lse = attn(q, k, v, causal, scale)
        T = q.shape[2]
        s = scale * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            s = np.where(np.tril(np.ones((T, T), dtype=bool)), s, -np.inf)
        assert np.allclose(lse, logsumexp(s, axis=-1), rtol=0, atol=1e-12)


def brute_force(q, k, v, causal, scale):
    """Full score matrix S, full probability matrix P, then P V (no tiling)."""
    T = q.shape[2]
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.tril(np.ones((T, T), dtype=bool)), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    p = e / l
    return np.einsum("bhij,bhjd->bhid", p, v), (m + np.log(l))[..., 0]


def pin_brute_force(attn):
    """Agreement with the brute-force full-matrix computation on tiny inputs."""
    for q, k, v, causal, scale in _random_cases():
        o, lse = attn(q, k, v, causal, scale)
        ob, lb = brute_force(q, k, v, causal, scale)
        assert np.allclose(o, ob, rtol=0, atol=1e-12) and np.allclose(lse, lb, rtol=0, atol=1e-12)


ALL_PINS = [
    pin_w1_three_token, pin_w2_four_scores, pin_w4_online_code,
    pin_zero_scores_running_mean, pin_ones_values, pin_causal_first_row,
    pin_identity_values_lower_triangular, pin_shift_invariance, pin_linear_in_values,
    pin_key_permutation, pin_large_scores_no_overflow, pin_torch_sdpa, pin_scipy_logsumexp,
    pin_brute_force,
]
