"""The backward oracle against its pins, its selected-rows entry and its size checks (CPU only)."""
import numpy as np
import pytest

import oracle
import pins_bwd


def _grad(q, k, v, do, causal, scale):
    return oracle.attention_bwd_f64(q, k, v, do, causal, scale)


@pytest.mark.parametrize("pin", pins_bwd.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_bwd_pin(pin):
    pin(_grad)


@pytest.mark.parametrize("shape", [(2, 4, 2, 13, 13, 8, True), (1, 3, 3, 6, 17, 5, True),
                                   (2, 2, 1, 9, 12, 4, False)])
def test_bwd_rows_match_full(shape):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    rng = np.random.default_rng(7)
    q, do = rng.standard_normal((B, Hq, Tq, d)), rng.standard_normal((B, Hq, Tq, d))
    k, v = rng.standard_normal((B, Hkv, Tk, d)), rng.standard_normal((B, Hkv, Tk, d))
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, do, causal, 0.37)
    qr = rng.choice(B * Hq * Tq, size=7, replace=False)
    kr = rng.choice(B * Hkv * Tk, size=6, replace=False)
    rq, rk, rv = oracle.attention_bwd_rows_f64(q, k, v, do, causal, 0.37, qr, kr)
    assert np.abs(rq - dq.reshape(-1, d)[qr]).max() <= 1e-13
    assert np.abs(rk - dk.reshape(-1, d)[kr]).max() <= 1e-13
    assert np.abs(rv - dv.reshape(-1, d)[kr]).max() <= 1e-13
    e = oracle.attention_bwd_rows_f64(q, k, v, do, causal, 0.37, [], [])
    assert e[0].shape == (0, d) and e[1].shape == (0, d)


def test_bwd_rejects_bad_sizes():
    q = np.zeros((1, 3, 4, 2))
    k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_bwd_f64(q, k, k, q, False, 1.0)      # 3 query heads over 2
    q = np.zeros((1, 2, 5, 2))
    k = np.zeros((1, 2, 4, 2))
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_f64(q, k, k, q, True, 1.0)       # causal with Tq > Tk
    with pytest.raises(ValueError):
        oracle.attention_bwd_f64(q, k, k, q[:, :, :4], False, 1.0)
    q = np.zeros((1, 2, 4, 2))
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_rows_f64(q, k, k, q, False, 1.0, [8], [])
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_rows_f64(q, k, k, q, False, 1.0, [], [-1])


def test_bwd_rows_given_d_is_the_identity_for_exact_o():
    """D_i = dO_i . O_i (O from the oracle forward) given explicitly reproduces the computed D."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, Tq, Tk, d = 1, 4, 2, 11, 11, 6
    q, do = rng.standard_normal((B, Hq, Tq, d)), rng.standard_normal((B, Hq, Tq, d))
    k, v = rng.standard_normal((B, Hkv, Tk, d)) * 2, rng.standard_normal((B, Hkv, Tk, d))
    o, _ = oracle.attention_f64(q, k, v, True, 0.6)
    D = np.einsum("bhid,bhid->bhi", do, o)
    qr, kr = np.arange(B * Hq * Tq), np.arange(B * Hkv * Tk)
    a = oracle.attention_bwd_rows_f64(q, k, v, do, True, 0.6, qr, kr)
    b = oracle.attention_bwd_rows_f64(q, k, v, do, True, 0.6, qr, kr, d_rows=D)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-12
    # and a perturbed D moves the gradients (the override is read)
    c = oracle.attention_bwd_rows_f64(q, k, v, do, True, 0.6, qr, kr, d_rows=D + 0.01)
    assert np.abs(c[0] - a[0]).max() > 1e-4 and np.abs(c[1] - a[1]).max() > 1e-4
    assert np.abs(c[2] - a[2]).max() <= 1e-12   # dV does not involve D
