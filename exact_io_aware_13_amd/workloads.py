"""Seeded synthetic workloads: attention shapes, input draws and row samples.

This module holds no attention arithmetic.  It draws Q, K, V values from a
seeded generator, rounds them to bf16 and picks sample rows; both the GPU path
and the CPU oracle consume exactly the bits it produces.

Shapes follow the model shapes the pages use: GPT-2 124M (12 heads of size 64,
named on "Flash Attention, tiled: exact attention without the T x T HBM
matrix", section "A three-token example"), GPT-2 medium (16 heads of size 64,
1,024 tokens, "FlashAttention and Fused Kernels: Attention Without the n x n
Matrix", "How much traffic it saves") and Llama 3.1 8B (32 heads of size 128,
the 32,768-token prompt of the same page's "Why it matters").  No dataset or
trained weights are involved: i.i.d. normal values stand in for activations.

Recipe: ``numpy.random.default_rng(seed)`` draws Q, then K, then V as float32
standard normals of shape (B, H, T, d).  For the spiky long-context workload it
then draws a Q-row mask and a K-row mask, each Bernoulli(0.01) per (b, h, t),
and multiplies the selected rows by 8 (a power of two, so exact in bf16).  The
values are then rounded to bf16 with round-to-nearest-even.  For the FP8
workloads the same float32 draw is divided by a per-tensor descale factor
(amax / 448) and rounded to OCP FP8 E4M3, ties to even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    B: int
    H: int
    T: int
    d: int
    causal: bool
    seed: int
    spikes: bool = False
    sampled_rows: bool = False   # parity on sampled rows instead of every row
    hkv: int = 0                 # key/value heads (0: one per query head)
    tk: int = 0                  # keys (0: T, the square problem)
    n_split: int = 1             # key splits for the split forward (None: the library's advice)
    fp8: bool = False            # inputs in FP8 E4M3 with per-tensor descale factors

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def Hkv(self) -> int:
        return self.hkv or self.H

    @property
    def Tk(self) -> int:
        return self.tk or self.T

    @property
    def shape(self):
        return (self.B, self.H, self.T, self.d)

    @property
    def kv_shape(self):
        return (self.B, self.Hkv, self.Tk, self.d)

    def flops(self) -> float:
        """Attention FLOPs: 4 d per visible (query, key) pair; for the square
        problem 4*B*H*T^2*d, halved for causal (metric convention)."""
        if self.Tk == self.T:
            f = 4.0 * self.B * self.H * self.T * self.T * self.d
            return f / 2.0 if self.causal else f
        if not self.causal:
            return 4.0 * self.B * self.H * self.T * self.Tk * self.d
        off = self.Tk - self.T   # query i sees i + off + 1 keys
        pairs = self.T * (off + 1) + self.T * (self.T - 1) / 2.0
        return 4.0 * self.B * self.H * pairs * self.d

    def algorithmic_bytes(self) -> int:
        """One read of Q, K, V (2 B/element, 1 B in FP8) and one write of O
        (2 B/element) plus lse (4 B/row)."""
        nq = self.B * self.H * self.T
        nkv = self.B * self.Hkv * self.Tk
        eb = 1 if self.fp8 else 2
        return nq * self.d * (eb + 2) + 2 * nkv * self.d * eb + 4 * nq


WORKLOADS = [
    Workload("c1", "causal B=1 H=1 T=128 d=64", 1, 1, 128, 64, True, seed=1),
    Workload("c2", "GPT-2-124M-shaped causal B=8 H=12 T=1024 d=64", 8, 12, 1024, 64, True, seed=2),
    Workload("c3nc", "GPT-2-medium-shaped non-causal B=16 H=16 T=1024 d=64", 16, 16, 1024, 64, False,
             seed=3),
    Workload("c3c", "GPT-2-medium-shaped causal B=16 H=16 T=1024 d=64", 16, 16, 1024, 64, True, seed=3),
    Workload("c4", "Llama-3.1-8B-shaped causal prefill B=1 H=32 T=8192 d=128", 1, 32, 8192, 128, True,
             seed=4),
    Workload("c5", "long-context spiky causal prefill B=1 H=32 T=32768 d=128", 1, 32, 32768, 128, True,
             seed=5, spikes=True, sampled_rows=True),
    # Llama 3.1 8B shares each key/value head among four query heads.
    Workload("gqa", "Llama-3.1-8B GQA causal prefill B=1 Hq=32 Hkv=8 T=8192 d=128", 1, 32, 8192, 128, True,
             seed=6, sampled_rows=True, hkv=8),
    Workload("decode", "Llama-3.1-8B GQA decode B=8 Hq=32 Hkv=8 Tq=1 Tk=32768 d=128, split keys", 8, 32, 1, 128,
             True, seed=7, hkv=8, tk=32768, n_split=None),
    Workload("decodefp8", "Llama-3.1-8B GQA decode B=8 Hq=32 Hkv=8 Tq=1 Tk=32768 d=128, split keys, FP8 E4M3 inputs",
             8, 32, 1, 128, True, seed=7, hkv=8, tk=32768, n_split=None, fp8=True),
    # The c4 shape and draw with FP8 E4M3 inputs (per-tensor descale factors).
    Workload("c4fp8", "Llama-3.1-8B-shaped causal prefill B=1 H=32 T=8192 d=128, FP8 E4M3 inputs", 1, 32, 8192,
             128, True, seed=4, sampled_rows=True, fp8=True),
]
BY_KEY = {w.key: w for w in WORKLOADS}

# The benchmarked workload: the Llama-3.1-8B-shaped causal prefill.
BENCH_KEY = "c4"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input values")
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float32 values (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_f32(shape, seed: int, spikes: bool = False):
    """Seeded float32 Q, K, V of ``shape`` = (B, H, T, d), drawn in that order."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(size=shape, dtype=np.float32)
    k = rng.standard_normal(size=shape, dtype=np.float32)
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if spikes:
        B, H, T, _ = shape
        q_mask = rng.random(size=(B, H, T)) < 0.01
        k_mask = rng.random(size=(B, H, T)) < 0.01
        q[q_mask] *= np.float32(8.0)
        k[k_mask] *= np.float32(8.0)
    return q, k, v


def draw_bf16(shape, seed: int, spikes: bool = False):
    """Seeded Q, K, V as bf16 bit patterns (uint16 arrays of ``shape``)."""
    q, k, v = draw_f32(shape, seed, spikes)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def workload_inputs(w: Workload):
    """The bf16 Q, K, V bits of a named workload.

    Square one-head-per-query-head workloads use ``draw_bf16``.  Others draw
    Q (B, Hq, Tq, d), then K and V (B, Hkv, Tk, d), from one generator in that
    order (no spikes)."""
    if w.kv_shape == w.shape:
        return draw_bf16(w.shape, w.seed, w.spikes)
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal(size=w.shape, dtype=np.float32)
    k = rng.standard_normal(size=w.kv_shape, dtype=np.float32)
    v = rng.standard_normal(size=w.kv_shape, dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


E4M3_MAX = 448.0


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round values to OCP FP8 E4M3 (round to nearest, ties to even), saturating
    at +-448; returns uint8 bits (sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 holds the subnormals m * 2^-9).  The sign is kept,
    also where the value rounds to zero (-0 is 0x80), as IEEE rounding does."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input values")
    a = np.abs(x)
    # binade exponent, at least -6 (the subnormals share the spacing of [2^-6, 2^-5))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = np.exp2(e - 3.0)
    r = np.minimum(np.rint(a / step) * step, E4M3_MAX)   # np.rint rounds ties to even
    # re-derive the fields of the rounded value (rounding may carry into the next binade)
    e2 = np.floor(np.log2(np.maximum(r, 2.0 ** -6)))
    sub = r < 2.0 ** -6
    m_sub = np.rint(r / 2.0 ** -9)
    m_nrm = np.rint(r / np.exp2(e2) * 8.0) - 8.0
    bits = np.where(sub, m_sub, (e2 + 7.0) * 8.0 + m_nrm).astype(np.uint8)
    return bits | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))


def e4m3_descale(x: np.ndarray) -> np.float32:
    """Per-tensor descale factor amax / 448 (fp32; 1 for an all-zero tensor)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    return np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)


def quantize_e4m3(x: np.ndarray):
    """(bits, descale) with x ~= descale * e4m3(bits): x / descale rounded to E4M3."""
    ds = e4m3_descale(x)
    return f32_to_e4m3_bits(np.asarray(x, dtype=np.float64) / np.float64(ds)), ds


def workload_inputs_fp8(w: Workload):
    """FP8 E4M3 Q, K, V of a workload: the same float32 draw as the bf16 inputs,
    each tensor divided by its descale factor and rounded to E4M3.  Returns
    ``(q8, k8, v8, (q_descale, k_descale, v_descale))``."""
    if w.kv_shape == w.shape:
        q, k, v = draw_f32(w.shape, w.seed, w.spikes)
    else:
        rng = np.random.default_rng(w.seed)
        q = rng.standard_normal(size=w.shape, dtype=np.float32)
        k = rng.standard_normal(size=w.kv_shape, dtype=np.float32)
        v = rng.standard_normal(size=w.kv_shape, dtype=np.float32)
    (q8, qd), (k8, kd), (v8, vd) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    return q8, k8, v8, (qd, kd, vd)


def workload_grad_output(w: Workload) -> np.ndarray:
    """The bf16 bits of the upstream gradient dO (shape of Q) for a backward run."""
    rng = np.random.default_rng(w.seed + 7919)
    return f32_to_bf16_bits(rng.standard_normal(size=w.shape, dtype=np.float32))


def spike_masks(shape, seed: int):
    """The (q_mask, k_mask) row masks ``draw_f32`` applies for spiky workloads."""
    rng = np.random.default_rng(seed)
    for _ in range(3):
        rng.standard_normal(size=shape, dtype=np.float32)
    B, H, T, _ = shape
    q_mask = rng.random(size=(B, H, T)) < 0.01
    k_mask = rng.random(size=(B, H, T)) < 0.01
    return q_mask, k_mask


def sample_rows(w: Workload, n_heads: int = 4, n_rows: int = 64, seed_offset: int = 1000,
                q_mask: np.ndarray | None = None):
    """Seeded sample of flat row indices ``(b*H + h)*T + i``.

    ``n_heads`` distinct (b, h) pairs, ``n_rows`` distinct rows each.  Every
    head always includes rows 0, 1, 63, 64, 127, 128 and T-1 (the first rows
    and the rows around 64- and 128-row tile boundaries), plus, when a spike
    mask is given, up to 8 of that head's spiked query rows.
    """
    rng = np.random.default_rng(w.seed + seed_offset)
    n_bh = w.B * w.H
    heads = rng.choice(n_bh, size=min(n_heads, n_bh), replace=False)
    out = []
    for bh in sorted(int(x) for x in heads):
        fixed = [i for i in (0, 1, 63, 64, 127, 128, w.T - 1) if 0 <= i < w.T]
        chosen = list(dict.fromkeys(fixed))
        if q_mask is not None:
            b, h = divmod(bh, w.H)
            spiked = np.flatnonzero(q_mask[b, h])
            for i in spiked[:8]:
                if int(i) not in chosen:
                    chosen.append(int(i))
        taken = set(chosen)
        rest = [i for i in range(w.T) if i not in taken]
        need = max(0, min(n_rows, w.T) - len(chosen))
        if need:
            chosen += [int(x) for x in rng.choice(rest, size=need, replace=False)]
        out += [bh * w.T + i for i in sorted(chosen[:n_rows])]
    return np.asarray(out, dtype=np.int64)
