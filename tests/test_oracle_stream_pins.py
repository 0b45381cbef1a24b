"""Pins of the oracle's streaming functions (generated tokens joining the cache).

The streaming state is the selection's whole 32-token groups packed plus a
residual window of exact tokens; every 32nd residual token packs the window as
the next group.  Pins: the split of a selection; streaming a token sequence
through appends and flushes gives the same packed bytes as packing the whole
sequence at once (group alignment, flush timing, residual contents); decode
over a cache whose groups dequantise exactly equals plain softmax attention
over the raw keys and values (brute force, written out here); with no residual
it equals decode over the packed cache alone.
"""
import math

import numpy as np
import pytest

import oracle



def test_stream_split():
    assert oracle.stream_split_ref(614) == (608, 6)
    assert oracle.stream_split_ref(32) == (32, 0)
    assert oracle.stream_split_ref(31) == (0, 31)
    assert oracle.stream_split_ref(6600) == (6592, 8)


def _tokens(rng, B, H, n, D):
    return rng.standard_normal((B, H, n, D)).astype(np.float32)


def test_streaming_equals_one_shot_pack():
    rng = np.random.default_rng(11)
    B, H, T, D = 2, 2, 200, 64
    k = _tokens(rng, B, H, T, D)
    v = _tokens(rng, B, H, T, D)
    idx = np.sort(np.stack([[rng.choice(T, 70, replace=False) for _ in range(H)] for _ in range(B)]), -1)
    st = oracle.stream_init_ref(k, v, idx)
    assert st["packed"]["k_codes"].shape[2] == 64 and st["k_res"].shape[2] == 6
    new_k = _tokens(rng, B, H, 60, D)
    new_v = _tokens(rng, B, H, 60, D)
    flushes = []
    for i in range(60):
        before = st["packed"]["k_codes"].shape[2]
        st = oracle.stream_append_ref(st, new_k[:, :, i], new_v[:, :, i])
        if st["packed"]["k_codes"].shape[2] != before:
            flushes.append(i)
    assert flushes == [25, 57]  # 6 + 26 = 32, then 32 more
    assert st["packed"]["k_codes"].shape[2] == 128 and st["k_res"].shape[2] == 2
    # the same tokens in order: the 70 selected, then the 60 generated
    seq_k = np.concatenate([np.take_along_axis(k, idx[..., None], 2), new_k], axis=2)
    seq_v = np.concatenate([np.take_along_axis(v, idx[..., None], 2), new_v], axis=2)
    one = oracle.quant_pack_ref(seq_k[:, :, :128], seq_v[:, :, :128])
    for key in one:
        assert np.array_equal(one[key], st["packed"][key]), key
    assert np.array_equal(st["k_res"], seq_k[:, :, 128:]) and np.array_equal(st["v_res"], seq_v[:, :, 128:])


def _exact_groups(rng, B, H, n, D, s=0.25, z=-0.5):
    """Values on the grid z + {0,1,2,3} s with every key group (32 tokens x 1
    channel) and value group (1 token x 32 channels) holding both extremes, so
    that scale = s, zero = z and the codes reproduce the values exactly."""
    codes = rng.integers(0, 4, size=(B, H, n, D))
    kc = codes.copy()
    for g0 in range(0, n, 32):  # key groups: both extremes in every channel
        kc[:, :, g0, :] = 0
        kc[:, :, g0 + 1, :] = 3
    vc = rng.integers(0, 4, size=(B, H, n, D))
    for c0 in range(0, D, 32):  # value groups: both extremes in every token
        vc[:, :, :, c0] = 0
        vc[:, :, :, c0 + 1] = 3
    return (z + s * kc).astype(np.float32), (z + s * vc).astype(np.float32)


def _softmax_attention(q, keys, vals, scale):
    keys = np.asarray(keys, np.float64)
    vals = np.asarray(vals, np.float64)
    B, Hq, D = q.shape
    Hkv = keys.shape[1]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            w = [math.exp(scale * float(np.dot(q[b, h], keys[b, g, t]))) for t in range(keys.shape[2])]
            tot = sum(w)
            for t in range(keys.shape[2]):
                out[b, h] += (w[t] / tot) * vals[b, g, t]
    return out


def test_stream_decode_brute_force_exact_groups():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D = 1, 4, 2, 64
    kx, vx = _exact_groups(rng, B, Hkv, 64, D)
    st = oracle.stream_init_ref(kx, vx, np.broadcast_to(np.arange(64), (B, Hkv, 64)))
    k_hat, v_hat = oracle.dequant_ref(st["packed"])
    assert np.array_equal(k_hat, kx) and np.array_equal(v_hat, vx)  # the grid values come back exactly
    extra_k = rng.standard_normal((B, Hkv, 5, D)).astype(np.float32)
    extra_v = rng.standard_normal((B, Hkv, 5, D)).astype(np.float32)
    for i in range(5):
        st = oracle.stream_append_ref(st, extra_k[:, :, i], extra_v[:, :, i])
    q = rng.standard_normal((B, Hq, D))
    got = oracle.stream_decode_ref(q, st)
    want = _softmax_attention(q, np.concatenate([kx, extra_k], 2), np.concatenate([vx, extra_v], 2), 1 / math.sqrt(D))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_stream_decode_residual_only_is_exact_attention():
    rng = np.random.default_rng(13)
    B, H, T, D = 2, 2, 40, 64
    k = _tokens(rng, B, H, T, D)
    v = _tokens(rng, B, H, T, D)
    idx = np.broadcast_to(np.arange(0, 40, 2), (B, H, 20))
    st = oracle.stream_init_ref(k, v, idx)
    assert st["packed"]["k_codes"].shape[2] == 0
    q = rng.standard_normal((B, H, D))
    want = _softmax_attention(q, k[:, :, ::2], v[:, :, ::2], 1 / math.sqrt(D))
    assert np.allclose(oracle.stream_decode_ref(q, st), want, rtol=1e-12, atol=1e-12)


def test_stream_decode_without_residual_is_packed_decode():
    rng = np.random.default_rng(14)
    B, Hq, Hkv, T, D = 1, 4, 2, 100, 64
    k = _tokens(rng, B, Hkv, T, D)
    v = _tokens(rng, B, Hkv, T, D)
    idx = np.sort(np.stack([[rng.choice(T, 64, replace=False) for _ in range(Hkv)] for _ in range(B)]), -1)
    st = oracle.stream_init_ref(k, v, idx)
    q = rng.standard_normal((B, Hq, D))
    assert np.array_equal(oracle.stream_decode_ref(q, st), oracle.decode_ref(q, st["packed"]))
