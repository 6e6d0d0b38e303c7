"""Oracle for the FP8 forward: exact attention of the dequantised inputs, and
the error the FP8 weights may add.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the CPU-baseline leg of the benchmark use it.

"FlashAttention and Fused Kernels: Attention Without the n x n Matrix" ("Four
generations") names an FP8 mode of FlashAttention-3 but gives no recipe.  The
reading taken here is the plainest one:

* Q, K and V arrive as OCP FP8 E4M3 values with one fp32 descale factor per
  tensor, so the operand that is meant is ``descale * e4m3`` (the E4M3 format
  is the one of the OCP 8-bit floating point specification: 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, exponent field 0 for the
  subnormals m * 2^-9, the all-ones pattern S.1111.111 for NaN, no infinity,
  largest finite value 448).
* The result the method must reach is the ordinary attention of those
  dequantised operands, the same definition as for bf16 inputs.  So
  ``attention_fp8_f64`` widens the bits exactly and calls the plain oracle.
* The FP8 forward also feeds the probability weights to the matrix product in
  E4M3.  That rounding is the one approximation; its effect is bounded per
  output element by ``pv_error_bound_rows`` and estimated in the mean square by
  ``pv_error_rms_rows``.

The bound.  Let w_j be the exact softmax weights of a row, O = sum_j w_j v_j,
and let the weights used be q_j = r_j + e_j where r_j = S w_j (S > 0 the sum of
the exact weights in the kernel's units) and e_j the E4M3 rounding error.  With
the row normalised by the sum of the used weights,

    O' - O = sum_j e_j (v_j - O) / sum_j q_j,

so |O' - O| <= sum_j |e_j| |v_j - O| / (S (1 - sum_j |e_j| / S)).  Rounding to
nearest E4M3 gives |e| <= 2^-4 r for r >= 2^-6 (3 mantissa bits) and
|e| <= min(2^-10, r) below (subnormal spacing 2^-9).  The weights are formed
as 2^3 * 2^(x_j - m) against a reference m that never exceeds the row max, so
the largest of them is at least 8 and S >= 8 Z with Z = sum_j exp(s_j - max s)
>= 1.  Hence |e_j| / S <= omega_j = max(2^-4 w_j, min(2^-13 / Z, w_j)).

Beyond the weights' rounding, the arithmetic of the FP8 matrix instruction
(v_mfma_f32_32x32x64_f8f6f4) enters: it sums its 64 products with an error of
up to KAPPA_MFMA times the largest product (2^-10.9 measured on MI355X over
random, equal-weight and cancelling operands; 2^-10 taken), and adds that sum
to its fp32 accumulator with one rounding.  This does not come from the pages;
it is the instruction's own precision.  In the PV product (one instruction per
64 keys) it adds at most KAPPA_MFMA (1 + 2^-4) (sum_j w_j |v_j| + |O|) to an
element (the product and the weight sum, each bounded by the sum over all keys
instead of per 64-key block).  In the scores (one instruction per 64 head-dim
values, at most two) it moves s_j by at most
delta_j = 2 KAPPA_MFMA |scale| max_k |q_k kk_jk| (plus fp32 rounding), which
moves every normalised weight by a factor within exp(+-2 max_j delta_j) and lse
by at most max_j delta_j (``score_error_rows``).  The fp32 accumulation over
the key blocks adds at most n 2^-24 sum_j w_j |v_j| for each of the two sums
(n the keys of the row), and the final bf16 store rounds with relative error
<= 2^-8.
"""
from __future__ import annotations

import numpy as np

from . import attention_f64, attention_rows_f64, _check4

U_FP8 = 2.0 ** -4        # unit roundoff of E4M3 (3 mantissa bits)
A_FP8 = 2.0 ** -13       # subnormal half-spacing 2^-10 over the smallest weight sum 8
KAPPA_MFMA = 2.0 ** -10  # FP8 matrix instruction: error of its 64-product sum / largest product
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def widen_e4m3(bits) -> np.ndarray:
    """OCP E4M3 bit patterns (uint8) -> float64, exactly; NaN patterns give NaN."""
    b = np.ascontiguousarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def dequantize(bits, descale) -> np.ndarray:
    """descale * e4m3(bits) in float64 (exact: 4 significant bits times an fp32)."""
    return widen_e4m3(bits) * np.float64(np.float32(descale))


def attention_fp8_f64(q8, k8, v8, descales, causal: bool, scale: float):
    """Exact attention of the dequantised FP8 operands; shapes and rules as
    ``attention_f64``.  Returns ``(o, lse)`` in float64."""
    qd, kd, vd = descales
    return attention_f64(dequantize(q8, qd), dequantize(k8, kd), dequantize(v8, vd), causal, scale)


def attention_fp8_rows_f64(q8, k8, v8, descales, causal: bool, scale: float, rows):
    """``attention_fp8_f64`` for selected flat rows ``(b*Hq + h)*Tq + i``."""
    qd, kd, vd = descales
    return attention_rows_f64(dequantize(q8, qd), dequantize(k8, kd), dequantize(v8, vd), causal, scale, rows)


def _row_scores(q, k, causal, scale, rows):
    """Per selected row: the visible scores s and the largest |q_k kk_jk| of each key."""
    _check4(q, k, k)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    off = Tk - Tq
    for r in np.asarray(rows, dtype=np.int64):
        bh, i = divmod(int(r), Tq)
        b, h = divmod(bh, Hq)
        n = min(Tk, i + off + 1) if causal else Tk
        kk = k[b, h // g, :n]
        yield scale * (kk @ q[b, h, i]), np.abs(kk * q[b, h, i]).max(axis=1), (b, h // g, n)


def score_error_rows(q, k, causal: bool, scale: float, rows, kappa: float = KAPPA_MFMA) -> np.ndarray:
    """Per selected row, a bound on how far the kernel's scores (and so its lse)
    may move: max_j of 2 kappa |scale| max_k |q_k kk_jk| plus fp32 rounding
    of the scaled score (module docstring; kappa = KAPPA_MFMA unless a caller
    asks how much of the bound the instruction's term is)."""
    out = []
    for s, pmax, _ in _row_scores(q, k, causal, scale, rows):
        out.append(float(np.max(2.0 * kappa * abs(scale) * pmax + 4.0 * U_F32 * np.abs(s))))
    return np.asarray(out)


def _row_terms(q, k, v, causal, scale, rows, kappa=KAPPA_MFMA):
    """Per selected row: the exact weights w, Z, O, the visible V rows and the score bound."""
    _check4(q, k, v)
    for s, pmax, (b, hk, n) in _row_scores(q, k, causal, scale, rows):
        vv = v[b, hk, :n]
        e = np.exp(s - s.max())
        z = e.sum()
        w = e / z
        delta = float(np.max(2.0 * kappa * abs(scale) * pmax + 4.0 * U_F32 * np.abs(s)))
        yield w, z, w @ vv, vv, delta


def pv_error_bound_rows(q, k, v, causal: bool, scale: float, rows, kappa: float = KAPPA_MFMA) -> np.ndarray:
    """Per-element bound (n, d) on |O_fp8 - O| for the selected rows of the
    dequantised problem (float64 operands), from the FP8 rounding of the
    weights, the FP8 matrix instruction's summation, the fp32 accumulation and
    the bf16 store (module docstring).  ``kappa`` is the instruction's term,
    KAPPA_MFMA unless a caller asks how much of the bound that term is."""
    out = []
    for w, z, o, vv, delta in _row_terms(q, k, v, causal, scale, rows, kappa):
        omega = np.maximum(U_FP8 * w, np.minimum(A_FP8 / z, w))
        big = omega.sum()
        dev = np.abs(vv - o)                       # (n, d)
        wv = w @ np.abs(vv)
        acc = 2.0 * len(w) * U_F32 * wv + kappa * (1.0 + U_FP8) * (wv + np.abs(o))
        shift = np.expm1(2.0 * delta) * (w @ dev)  # the scores' error moves the weights
        b = (omega @ dev + acc + shift) / (1.0 - big) if big < 0.5 else np.full(o.shape, np.inf)
        out.append(b + U_BF16 * (np.abs(o) + b))
    return np.asarray(out)


def pv_error_rms_rows(q, k, v, causal: bool, scale: float, rows) -> float:
    """Root of the summed squared error expected from the weights' rounding over
    the selected rows: each weight's relative error taken as uniform on
    [-2^-4, 2^-4] (variance 2^-8 / 3) and independent, plus the bf16 store's
    (relative variance 2^-16 / 3)."""
    tot = 0.0
    for w, _z, o, vv, _delta in _row_terms(q, k, v, causal, scale, rows):
        dev = vv - o
        tot += (U_FP8 ** 2 / 3.0) * float(np.sum((w[:, None] * dev) ** 2))
        tot += (U_BF16 ** 2 / 3.0) * float(np.sum(o ** 2))
    return float(np.sqrt(tot))
