"""The backward pins have teeth: plausible mistakes planted in a full-matrix
numpy backward (CPU only) must each fail at least one pin."""
import numpy as np
import pytest

import pins_bwd


def _make(no_D=False, D_sign=1.0, dq_scale=True, dk_scale=True, dv_transposed=True, dq_uses_dsT=False,
          mask_shift=0, D_unnormalised=False, gqa_first_only=False, dk_uses_v=False, dv_uses_ds=False,
          swap_dk_dv=False, softmax_unscaled=False, dq_uses_v=False):
    def grad(q, k, v, do, causal, scale):
        B, Hq, Tq, d = q.shape
        Hkv, Tk = k.shape[1], k.shape[2]
        g = Hq // Hkv
        kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
        s = (1.0 if softmax_unscaled else scale) * np.einsum("bhid,bhjd->bhij", q, kr)
        vis = np.ones((Tq, Tk), dtype=bool)
        if causal:
            vis = np.arange(Tk)[None, :] <= np.arange(Tq)[:, None] + (Tk - Tq) + mask_shift
            vis[:, 0] = True
        s = np.where(vis, s, -np.inf)
        e = np.exp(s - s.max(axis=-1, keepdims=True))
        p = e / e.sum(axis=-1, keepdims=True)
        dp = np.einsum("bhid,bhjd->bhij", do, vr)
        D = np.sum((e if D_unnormalised else p) * dp, axis=-1, keepdims=True)
        ds = p * dp if no_D else p * (dp - D_sign * D)
        kq = vr if dq_uses_v else kr
        if dq_uses_dsT and Tq == Tk:
            dq = np.einsum("bhji,bhjd->bhid", ds, kq)
        else:
            dq = np.einsum("bhij,bhjd->bhid", ds, kq)
        dq = dq * (scale if dq_scale else 1.0)
        dkr = np.einsum("bhij,bhid->bhjd", ds, v.repeat(g, axis=1)[:, :, :Tq] if (dk_uses_v and Tq == Tk) else q)
        dkr = dkr * (scale if dk_scale else 1.0)
        if dv_uses_ds:
            dvr = np.einsum("bhij,bhid->bhjd", ds, do)
        elif dv_transposed or Tq != Tk:
            dvr = np.einsum("bhij,bhid->bhjd", p, do)
        else:
            dvr = np.einsum("bhji,bhid->bhjd", p, do)
        if gqa_first_only:
            dk = dkr.reshape(B, Hkv, g, Tk, d)[:, :, 0]
            dv = dvr.reshape(B, Hkv, g, Tk, d)[:, :, 0]
        else:
            dk = dkr.reshape(B, Hkv, g, Tk, d).sum(axis=2)
            dv = dvr.reshape(B, Hkv, g, Tk, d).sum(axis=2)
        if swap_dk_dv:
            dk, dv = dv, dk
        return dq, dk, dv
    return grad


MUTANTS = {
    "no_softmax_jacobian_term": _make(no_D=True),
    "jacobian_term_sign": _make(D_sign=-1.0),
    "dq_without_scale": _make(dq_scale=False),
    "dk_without_scale": _make(dk_scale=False),
    "dv_with_P_untransposed": _make(dv_transposed=False),
    "dq_with_dS_transposed": _make(dq_uses_dsT=True),
    "causal_excludes_diagonal": _make(mask_shift=-1),
    "causal_sees_one_future_key": _make(mask_shift=1),
    "jacobian_term_unnormalised": _make(D_unnormalised=True),
    "gqa_first_head_only": _make(gqa_first_only=True),
    "dk_from_values": _make(dk_uses_v=True),
    "dv_from_dS": _make(dv_uses_ds=True),
    "dk_dv_swapped": _make(swap_dk_dv=True),
    "softmax_without_scale": _make(softmax_unscaled=True),
    "dq_from_values": _make(dq_uses_v=True),
}


def _fails_some_pin(grad):
    failed = []
    for pin in pins_bwd.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(grad)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(name):
    assert _fails_some_pin(MUTANTS[name]), f"mutant {name} passed every pin"


def test_bwd_unmutated_passes():
    assert _fails_some_pin(_make()) == []
