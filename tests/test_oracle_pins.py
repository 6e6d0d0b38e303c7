"""The CPU oracle against its pins (worked examples, closed forms, invariants,
library routines, brute force).  No GPU involved."""
import math

import numpy as np
import pytest

import oracle
from oracle import online
import pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    pin(oracle.attention_f64)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_online_model_passes_pin(pin):
    """The tiled recurrence (block 3) passes the same pins as the definition."""
    pin(lambda q, k, v, c, s: online.attention_online_f64(q, k, v, c, s, block=3))


def test_w4_online_matches_full_to_machine_precision():
    """inference-learning-path section 4: online (block 2) equals full softmax, diff ~1e-16."""
    g = pins.golden("w4_online_softmax_code.json")
    K = np.asarray(g["K"]); V = np.asarray(g["V"]); T = K.shape[0]
    q = np.tile(np.asarray(g["q"]), (T, 1))[None, None]
    o_full, l_full = oracle.attention_f64(q, K[None, None], V[None, None], False, g["scale"])
    o_on, l_on = online.attention_online_f64(q, K[None, None], V[None, None], False, g["scale"],
                                             block=g["online_block"])
    assert np.max(np.abs(o_full - o_on)) <= 10 * g["printed_max_abs_diff"]
    assert np.max(np.abs(l_full - l_on)) <= 1e-14


def test_w5_max_change_states():
    """joelfernandes.org 'What happens when the maximum changes': the (m, l, o) states."""
    g = pins.golden("w5_max_change.json")
    st = online.RowState(3)
    V = np.eye(3)
    st.update(np.asarray(g["tiles"][0]), V[0:2])
    assert st.m == g["after_tile1"]["m"]
    assert abs(st.l - (math.exp(-1) + 1)) <= 1e-15
    assert np.allclose(st.o, [math.exp(-1), 1.0, 0.0], rtol=0, atol=1e-15)
    m_old = st.m
    st.update(np.asarray(g["tiles"][1]), V[2:3])
    assert st.m == g["after_tile2"]["m"]
    assert abs(math.exp(m_old - st.m) - math.exp(-2)) <= 1e-16
    assert abs(st.l - (math.exp(-2) * (math.exp(-1) + 1) + 1)) <= 1e-15
    assert np.allclose(st.o, [math.exp(-3), math.exp(-2), 1.0], rtol=0, atol=1e-15)


def test_w1_row2_two_tiles():
    """joelfernandes.org: row 2 of the three-token example over tiles {0,1} then {2}."""
    g = pins.golden("w1_three_token_causal.json")
    V = np.asarray(g["v"])
    st = online.RowState(2)
    st.update(np.zeros(2), V[0:2])
    a = g["online_row2"]["after_tile1"]
    assert (st.m, st.l) == (a["m"], a["l"]) and np.array_equal(st.o, a["o"])
    st.update(np.zeros(1), V[2:3])
    b = g["online_row2"]["after_tile2"]
    assert (st.m, st.l) == (b["m"], b["l"]) and np.array_equal(st.o, b["o"])
    pins._printed(st.output(), g["Y"][2], g["Y_printed_decimals"])


def test_w3_split_combine():
    """vidyal.ai Step 4: two blocks (max 2, sum 1.368, out 12.69) and (4, 1.368, 32.69) combine to 30.31."""
    g = pins.golden("w2_four_scores.json")
    s = np.asarray(g["scores"]); v = np.asarray(g["values"])[:, None]
    a = online.RowState(1); a.update(s[:2], v[:2])
    b = online.RowState(1); b.update(s[2:], v[2:])
    c = online.combine([a, b])
    pins._printed(math.exp(a.m - c.m), g["combine"]["rescale"], 3)
    pins._printed(c.l, g["combine"]["denominator"], 3)
    pins._printed(c.output()[0], g["combine"]["result"], 2)


@pytest.mark.parametrize("block", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_tile_size_does_not_change_result(block, causal):
    """inference-learning-path section 4: the tile size is a schedule, not an approximation."""
    rng = np.random.default_rng(20 + block)
    q, k, v = (rng.standard_normal((1, 2, 40, 8)) for _ in range(3))
    o, l = oracle.attention_f64(q, k, v, causal, 0.35)
    oo, lo = online.attention_online_f64(q, k, v, causal, 0.35, block=block)
    assert np.max(np.abs(o - oo)) <= 1e-14 and np.max(np.abs(l - lo)) <= 1e-14


def test_rows_entry_matches_full():
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((2, 3, 50, 16)) for _ in range(3))
    o, l = oracle.attention_f64(q, k, v, True, 0.25)
    rows = np.array([0, 1, 49, 50, 123, 299], dtype=np.int64)
    orow, lrow = oracle.attention_rows_f64(q, k, v, True, 0.25, rows)
    assert np.array_equal(orow, o.reshape(-1, 16)[rows])
    assert np.array_equal(lrow, l.reshape(-1)[rows])


def test_oracle_rejects_bad_sizes():
    z = np.zeros((1, 1, 0, 4))
    with pytest.raises(RuntimeError):
        oracle.attention_f64(z, z, z, True, 1.0)
    q = np.zeros((1, 1, 4, 4))
    with pytest.raises(RuntimeError):
        oracle.attention_rows_f64(q, q, q, True, 1.0, np.array([4]))


def test_widen_bf16_exact():
    bits = np.array([0x0000, 0x3F80, 0xBF80, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    x = oracle.widen_bf16(bits)
    assert x.dtype == np.float64
    assert list(x[:3]) == [0.0, 1.0, -1.0]
    assert x[3] == 3.140625
