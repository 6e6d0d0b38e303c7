"""The oracle's general entry (grouped heads, Tq != Tk) against its pins, and
plausible mistakes in a numpy version of it that the pins must catch."""
import numpy as np
import pytest

import oracle
import pins_general as pg


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", pg.ALL_GENERAL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_general_pin(pin):
    pin(oracle.attention_f64)


def test_general_rows_entry_matches_full():
    rng = np.random.default_rng(41)
    q, k, v = rng.standard_normal((2, 6, 9, 8)), rng.standard_normal((2, 3, 20, 8)), rng.standard_normal((2, 3, 20, 8))
    o, lse = oracle.attention_f64(q, k, v, True, 0.5)
    rows = np.array([0, 5, 9 * 6 - 1, 9 * 7 + 3, 2 * 6 * 9 - 1])
    orow, lrow = oracle.attention_rows_f64(q, k, v, True, 0.5, rows)
    assert np.array_equal(orow, o.reshape(-1, 8)[rows]) and np.array_equal(lrow, lse.reshape(-1)[rows])


def test_general_rejects_bad_sizes():
    q, k = np.zeros((1, 3, 4, 2)), np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_f64(q, k, k, False, 1.0)          # 3 query heads over 2 kv heads
    q, k = np.zeros((1, 2, 6, 2)), np.zeros((1, 2, 4, 2))
    with pytest.raises(RuntimeError):
        oracle.attention_f64(q, k, k, True, 1.0)           # causal with more queries than keys


def _general(q, k, v, causal, scale, head_map="group", align="bottom"):
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    idx = np.arange(Hq) // g if head_map == "group" else np.arange(Hq) % Hkv
    kk, vv = k[:, idx], v[:, idx]
    s = scale * np.einsum("bhid,bhjd->bhij", q, kk)
    if causal:
        off = Tk - Tq if align == "bottom" else 0
        s = np.where(np.ones((Tq, Tk), dtype=bool) & (np.arange(Tk)[None] <= np.arange(Tq)[:, None] + off), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return np.einsum("bhij,bhjd->bhid", e / l, vv), (m + np.log(l))[..., 0]


MUTANTS = {
    "heads_interleaved_not_grouped": lambda q, k, v, c, s: _general(q, k, v, c, s, head_map="mod"),
    "causal_aligned_top_left": lambda q, k, v, c, s: _general(q, k, v, c, s, align="top"),
}


def test_numpy_general_passes():
    for pin in pg.ALL_GENERAL_PINS:
        pin(_general)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_general_pins_catch_mutant(name):
    failed = []
    for pin in pg.ALL_GENERAL_PINS:
        try:
            pin(MUTANTS[name])
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every general pin"
