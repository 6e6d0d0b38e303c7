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
