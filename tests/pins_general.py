"""Pins for the general problem: grouped key/value heads and Tq != Tk.

Each pin takes ``attn(q, k, v, causal, scale) -> (o, lse)`` with q of shape
(B, Hq, Tq, d) and k, v of shape (B, Hkv, Tk, d), and checks it against
something other than itself:

* grouped heads: query head h reads key/value head h // (Hq // Hkv), the
  consecutive grouping of "FlashAttention and Fused Kernels: Attention Without
  the n x n Matrix", Step 4 (Llama 3.1 8B: four query heads per key/value head);
  checked against explicit replication of the key/value heads and against
  torch's ``enable_gqa`` attention;
* Tq != Tk with the causal rule of "Flash Attention, tiled: exact attention
  without the T x T HBM matrix" ("Ordinary causal attention") applied to query
  rows that are the last Tq positions of the sequence: query i sees keys
  j <= i + Tk - Tq; checked as the tail of the square problem, against an
  explicit-mask library call, and for the decode row (Tq = 1), which sees
  every key.
"""
import numpy as np


def _rand(rng, *shape, s=1.3):
    return rng.standard_normal(shape) * s


def pin_gqa_is_replicated_mha(attn):
    """Grouped heads equal the one-head-per-query-head problem with K, V repeated per group."""
    rng = np.random.default_rng(31)
    for (B, Hq, Hkv, T, d) in ((2, 6, 2, 13, 8), (1, 8, 1, 9, 4), (1, 4, 4, 7, 5)):
        q, k, v = _rand(rng, B, Hq, T, d), _rand(rng, B, Hkv, T, d), _rand(rng, B, Hkv, T, d)
        g = Hq // Hkv
        kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
        for causal in (True, False):
            o, lse = attn(q, k, v, causal, 0.4)
            o1, lse1 = attn(q, kr, vr, causal, 0.4)
            assert np.allclose(o, o1, rtol=0, atol=1e-13) and np.allclose(lse, lse1, rtol=0, atol=1e-13)


def pin_gqa_torch(attn):
    """torch's float64 CPU attention with enable_gqa computes the same O."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(32)
    B, Hq, Hkv, T, d = 2, 8, 2, 11, 6
    q, k, v = _rand(rng, B, Hq, T, d), _rand(rng, B, Hkv, T, d), _rand(rng, B, Hkv, T, d)
    for causal in (True, False):
        o, _ = attn(q, k, v, causal, 0.3)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             is_causal=causal, scale=0.3, enable_gqa=True).numpy()
        assert np.allclose(o, ref, rtol=0, atol=1e-12), np.abs(o - ref).max()


def pin_short_queries_are_the_tail(attn):
    """Tq < Tk causal rows equal the last Tq rows of the square causal problem."""
    rng = np.random.default_rng(33)
    B, H, Tk, d = 2, 3, 17, 8
    k, v = _rand(rng, B, H, Tk, d), _rand(rng, B, H, Tk, d)
    for Tq in (1, 5, 16, 17):
        q_full = _rand(rng, B, H, Tk, d)
        o_full, lse_full = attn(q_full, k, v, True, 0.5)
        o, lse = attn(q_full[:, :, Tk - Tq:], k, v, True, 0.5)
        assert np.allclose(o, o_full[:, :, Tk - Tq:], rtol=0, atol=1e-13)
        assert np.allclose(lse, lse_full[:, :, Tk - Tq:], rtol=0, atol=1e-13)


def pin_rect_masked_library(attn):
    """torch's float64 attention with the explicit mask j <= i + Tk - Tq, and unmasked for Tq != Tk."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(34)
    B, Hq, Hkv, d = 1, 4, 2, 8
    for Tq, Tk in ((3, 10), (10, 10), (7, 64)):
        q, k, v = _rand(rng, B, Hq, Tq, d), _rand(rng, B, Hkv, Tk, d), _rand(rng, B, Hkv, Tk, d)
        mask = torch.ones(Tq, Tk, dtype=torch.bool).tril(diagonal=Tk - Tq)
        for causal in (True, False):
            o, _ = attn(q, k, v, causal, 0.6)
            ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                                 attn_mask=mask if causal else None, scale=0.6,
                                                 enable_gqa=True).numpy()
            assert np.allclose(o, ref, rtol=0, atol=1e-12), (Tq, Tk, causal, np.abs(o - ref).max())
    # queries longer than keys are allowed without the mask
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 5, 4), _rand(rng, 1, 2, 5, 4)
    o, _ = attn(q, k, v, False, 0.6)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         scale=0.6).numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-12)


def pin_decode_row_sees_every_key(attn):
    """One query row against Tk keys: causal and unmasked agree, lse = logsumexp of the whole score row."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(35)
    B, Hq, Hkv, Tk, d = 2, 4, 1, 40, 8
    q, k, v = _rand(rng, B, Hq, 1, d), _rand(rng, B, Hkv, Tk, d), _rand(rng, B, Hkv, Tk, d)
    oc, lc = attn(q, k, v, True, 0.7)
    on, ln = attn(q, k, v, False, 0.7)
    assert np.allclose(oc, on, rtol=0, atol=1e-14) and np.allclose(lc, ln, rtol=0, atol=1e-14)
    s = 0.7 * np.einsum("bhd,bjd->bhj", q[:, :, 0], k[:, 0])
    assert np.allclose(lc[:, :, 0], logsumexp(s, axis=-1), rtol=0, atol=1e-12)


ALL_GENERAL_PINS = [pin_gqa_is_replicated_mha, pin_gqa_torch, pin_short_queries_are_the_tail,
                    pin_rect_masked_library, pin_decode_row_sees_every_key]
