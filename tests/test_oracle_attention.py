"""Pins of the oracle's attention, O = softmax(Q K^T / sqrt(d)) V (Lynx
paper, Section 2.1), over reconstructed bf16 K^ and V^ with grouped-query
heads and the causal tail of a verification batch."""
import math

import numpy as np
import torch

import oracle
from progressive_kv_transfer_amd import kvgen


def bits(t):
    return kvgen.bf16_bits(t)


def f32(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator()
    g.manual_seed(seed)
    return bits((torch.randn(shape, generator=g) * scale).to(torch.bfloat16))


def test_equal_keys_give_mean_of_values():
    """Identical keys make the softmax uniform: the output is the plain mean
    of the visible values."""
    ctx, nkv, d = 300, 2, 128
    k1 = _rand_bf16((1, nkv, d), 1)
    k = np.repeat(k1, ctx, axis=0)
    v = _rand_bf16((ctx, nkv, d), 2)
    q = _rand_bf16((1, 8, d), 3)
    o = oracle.attention(q, k, v, 1 / math.sqrt(d), False)
    for h in range(8):
        np.testing.assert_allclose(o[0, h], f32(v)[:, h // 4].mean(0),
                                   rtol=0, atol=1e-12)


def test_single_token_context():
    """With one visible token the output is that token's value."""
    d = 128
    q = _rand_bf16((1, 4, d), 4)
    k = _rand_bf16((1, 1, d), 5, 30.0)
    v = _rand_bf16((1, 1, d), 6)
    o = oracle.attention(q, k, v, 0.1, False)
    for h in range(4):
        assert np.array_equal(o[0, h], f32(v)[0, 0])


def test_matches_numpy_softmax_with_gqa_mapping():
    """Against an independent numpy evaluation; query head h must read KV
    head h // (n_qh / n_kvh) (a different mapping would not match)."""
    ctx, nq, nkv, d = 777, 8, 2, 128
    q = _rand_bf16((2, nq, d), 7)
    k = _rand_bf16((ctx, nkv, d), 8, 2.0)
    v = _rand_bf16((ctx, nkv, d), 9)
    sc = 1 / math.sqrt(d)
    o = oracle.attention(q, k, v, sc, False, threads=2)
    qf, kf, vf = f32(q), f32(k), f32(v)
    for r in range(2):
        for h in range(nq):
            s = kf[:, h // 4] @ qf[r, h] * sc
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ vf[:, h // 4]
            np.testing.assert_allclose(o[r, h], ref, rtol=1e-10, atol=1e-12)
            wrong = kf[:, h % nkv] @ qf[r, h] * sc
            if h % nkv != h // 4:
                pw = np.exp(wrong - wrong.max())
                assert not np.allclose(o[r, h], (pw / pw.sum()) @ vf[:, h % nkv])


def test_causal_tail_equals_truncated_context():
    """Query row r of a T-token verification batch sees positions
    0 .. ctx - T + r: it equals non-causal attention over that prefix."""
    ctx, T, nq, nkv, d = 500, 8, 4, 1, 128
    q = _rand_bf16((T, nq, d), 10)
    k = _rand_bf16((ctx, nkv, d), 11)
    v = _rand_bf16((ctx, nkv, d), 12)
    sc = 1 / math.sqrt(d)
    o = oracle.attention(q, k, v, sc, True)
    for r in range(T):
        vis = ctx - T + r + 1
        ref = oracle.attention(q[r:r + 1], k[:vis], v[:vis], sc, False)
        assert np.array_equal(o[r], ref[0])
    # rows differ only because of the tail positions
    o_nc = oracle.attention(q, k, v, sc, False)
    assert np.array_equal(o[T - 1], o_nc[T - 1])
    assert not np.array_equal(o[0], o_nc[0])
