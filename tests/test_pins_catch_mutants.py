"""The pins have teeth: plausible mistakes planted in an oracle-like CPU
implementation must each fail at least one pin.  Everything here runs on the
CPU; the mutants are small numpy variants of the full-matrix computation."""
import numpy as np
import pytest

import pins


def _scores(q, k, scale):
    return scale * np.einsum("bhid,bhjd->bhij", q, k)


def _mask(T, causal, offset=0, upper=False):
    if not causal:
        return np.ones((T, T), dtype=bool)
    m = np.tril(np.ones((T, T), dtype=bool), offset)
    return m.T if upper else m


def _make(score_fn=None, mask_fn=None, no_max=False, norm=True, lse_mode="nat",
          pv="normal", mask_after=False, drop_last=False, rescale_sign=False):
    def attn(q, k, v, causal, scale):
        T = q.shape[2]
        s = score_fn(q, k, v, scale) if score_fn else _scores(q, k, scale)
        vis = mask_fn(T, causal) if mask_fn else _mask(T, causal)
        if drop_last:
            vis = vis.copy(); vis[:, T - 1] = False; vis[np.arange(T), np.arange(T)] |= (T == 1)
        if not mask_after:
            s = np.where(vis, s, -np.inf)
        m = np.zeros(s.shape[:-1] + (1,)) if no_max else np.max(s, axis=-1, keepdims=True)
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(s - m)
            if mask_after:
                e = np.where(vis, e, 0.0)
                l = np.sum(np.exp(s - m), axis=-1, keepdims=True)
            else:
                l = np.sum(e, axis=-1, keepdims=True)
            if rescale_sign:
                e = e * np.exp(2 * (m - np.max(s, axis=-1, keepdims=True)) + 0.01 * (s - m))
            p = e / l if norm else e
            if pv == "transposed":
                o = np.einsum("bhji,bhjd->bhid", p, v)
            else:
                o = np.einsum("bhij,bhjd->bhid", p, v)
            if lse_mode == "nat":
                lse = (m + np.log(l))[..., 0]
            elif lse_mode == "no_max":
                lse = np.log(l)[..., 0]
            else:
                lse = ((m + np.log(l)) / np.log(2.0))[..., 0]
        return o, lse
    return attn


MUTANTS = {
    "causal_excludes_diagonal": _make(mask_fn=lambda T, c: _mask(T, c, offset=-1)),
    "causal_sees_one_future_key": _make(mask_fn=lambda T, c: _mask(T, c, offset=1)),
    "causal_mask_transposed": _make(mask_fn=lambda T, c: _mask(T, c, upper=True)),
    "no_max_subtraction": _make(no_max=True),
    "keys_replaced_by_values": _make(score_fn=lambda q, k, v, s: _scores(q, v, s)),
    "scale_ignored": _make(score_fn=lambda q, k, v, s: _scores(q, k, 1.0)),
    "scale_squared": _make(score_fn=lambda q, k, v, s: _scores(q, k, s * s)),
    "no_normalisation": _make(norm=False),
    "lse_without_max": _make(lse_mode="no_max"),
    "lse_base2": _make(lse_mode="log2"),
    "probabilities_transposed": _make(pv="transposed"),
    "mask_after_softmax": _make(mask_after=True),
    "last_key_dropped": _make(drop_last=True),
    "stale_rescale_factor": _make(rescale_sign=True),
    "query_key_swapped_dims": _make(score_fn=lambda q, k, v, s: s * np.einsum("bhid,bhjd->bhij", k, q)),
}


def _fails_some_pin(attn):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(attn)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failed = _fails_some_pin(MUTANTS[name])
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_passes():
    assert _fails_some_pin(_make()) == []
