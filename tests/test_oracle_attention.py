"""Pins for the oracle's dual-cache attention (CPU only).

Each pin comes from outside the oracle: a library routine (torch SDPA in
float64 on the CPU), closed forms (one key, two keys, zero query, equal keys)
and invariants that non-causal softmax attention must satisfy (key
permutation, value scaling/shift, ragged-prefix padding never read).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attend, dual_cache_kv


def _rand(rng, B, H, D, L, P, S):
    q = rng.standard_normal((B, L, H, D))
    kp = rng.standard_normal((B, H, P, D)); vp = rng.standard_normal((B, H, P, D))
    kb = rng.standard_normal((B, H, L, D)); vb = rng.standard_normal((B, H, L, D))
    ks = rng.standard_normal((B, H, S, D)); vs = rng.standard_normal((B, H, S, D))
    return q, kp, vp, kb, vb, ks, vs


def _sdpa(q, K, V):
    # q [L][D], K/V [T][D] -> torch's non-causal scaled_dot_product_attention in float64
    with torch.no_grad():
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], is_causal=False)
    return o[0, 0].numpy()


@pytest.mark.parametrize("B,H,D,L,P,S", [(1, 2, 64, 16, 0, 0), (2, 3, 64, 8, 40, 24), (1, 1, 128, 32, 100, 0)])
def test_matches_torch_sdpa(B, H, D, L, P, S):
    rng = np.random.default_rng(1)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, B, H, D, L, P, S)
    pl = np.full(B, P)
    o = attend(q, kp, vp, kb, vb, ks, vs, pl)
    for b in range(B):
        for h in range(H):
            K = np.concatenate([kp[b, h], kb[b, h], ks[b, h]])
            V = np.concatenate([vp[b, h], vb[b, h], vs[b, h]])
            np.testing.assert_allclose(o[b, :, h], _sdpa(q[b, :, h], K, V), rtol=1e-12, atol=1e-12)


def test_block_only_is_plain_noncausal_sdpa():
    # prefix and suffix empty: the block attends to itself, all positions, no mask
    rng = np.random.default_rng(2)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, 1, 2, 64, 12, 0, 0)
    o = attend(q, kp, vp, kb, vb, ks, vs, np.zeros(1, int))
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h], _sdpa(q[0, :, h], kb[0, h], vb[0, h]), rtol=1e-12, atol=1e-12)
    # the last query must see the first key: causal masking would break this
    with torch.no_grad():
        oc = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, :, 0])[None, None], torch.from_numpy(kb[0, 0])[None, None],
            torch.from_numpy(vb[0, 0])[None, None], is_causal=True)[0, 0].numpy()
    assert np.abs(o[0, 0, 0] - oc[0]).max() > 1e-3


def test_single_key_returns_its_value():
    rng = np.random.default_rng(3)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, 1, 1, 64, 1, 0, 0)
    o = attend(q, kp, vp, kb, vb, ks, vs, np.zeros(1, int))
    np.testing.assert_allclose(o[0, 0, 0], vb[0, 0, 0], rtol=0, atol=1e-15)


def test_two_keys_logistic_closed_form():
    rng = np.random.default_rng(4)
    D = 64
    q = rng.standard_normal((1, 1, 1, D))
    kp = rng.standard_normal((1, 1, 1, D)); vp = rng.standard_normal((1, 1, 1, D))
    kb = rng.standard_normal((1, 1, 1, D)); vb = rng.standard_normal((1, 1, 1, D))
    ks = np.zeros((1, 1, 0, D)); vs = np.zeros((1, 1, 0, D))
    o = attend(q, kp, vp, kb, vb, ks, vs, np.ones(1, int))
    s1 = float(q[0, 0, 0] @ kp[0, 0, 0]) / math.sqrt(D)
    s2 = float(q[0, 0, 0] @ kb[0, 0, 0]) / math.sqrt(D)
    w1 = 1.0 / (1.0 + math.exp(s2 - s1))
    np.testing.assert_allclose(o[0, 0, 0], w1 * vp[0, 0, 0] + (1 - w1) * vb[0, 0, 0], rtol=1e-12, atol=1e-14)


def test_zero_query_averages_all_values():
    rng = np.random.default_rng(5)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, 1, 2, 64, 4, 10, 6)
    q[:] = 0.0
    o = attend(q, kp, vp, kb, vb, ks, vs, np.full(1, 10))
    for h in range(2):
        mean = np.concatenate([vp[0, h], vb[0, h], vs[0, h]]).mean(axis=0)
        for l in range(4):
            np.testing.assert_allclose(o[0, l, h], mean, rtol=1e-12, atol=1e-14)


def test_equal_keys_average_values():
    rng = np.random.default_rng(6)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, 1, 1, 64, 3, 5, 7)
    k = rng.standard_normal(64)
    kp[:] = k; kb[:] = k; ks[:] = k
    o = attend(q, kp, vp, kb, vb, ks, vs, np.full(1, 5))
    mean = np.concatenate([vp[0, 0], vb[0, 0], vs[0, 0]]).mean(axis=0)
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(mean, (3, 64)), rtol=1e-12, atol=1e-14)


def test_key_permutation_across_segments_is_invariant():
    # non-causal attention is a function of the key/value multiset: moving keys
    # between prefix, block and suffix (same total) must not change anything
    rng = np.random.default_rng(7)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, 1, 2, 64, 8, 20, 12)
    o = attend(q, kp, vp, kb, vb, ks, vs, np.full(1, 20))
    for h in range(2):
        K, V = dual_cache_kv(kp, vp, kb, vb, ks, vs, 0, h, 20)
        perm = rng.permutation(K.shape[0])
        K2, V2 = K[perm], V[perm]
        kp[0, h], kb[0, h], ks[0, h] = K2[:20], K2[20:28], K2[28:]
        vp[0, h], vb[0, h], vs[0, h] = V2[:20], V2[20:28], V2[28:]
    o2 = attend(q, kp, vp, kb, vb, ks, vs, np.full(1, 20))
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-14)


def test_value_scaling_and_shift():
    rng = np.random.default_rng(8)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, 1, 1, 64, 4, 9, 3)
    pl = np.full(1, 9)
    o = attend(q, kp, vp, kb, vb, ks, vs, pl)
    o2 = attend(q, kp, 3 * vp, kb, 3 * vb, ks, 3 * vs, pl)
    np.testing.assert_allclose(o2, 3 * o, rtol=1e-12, atol=1e-13)
    c = rng.standard_normal(64)
    o3 = attend(q, kp, vp + c, kb, vb + c, ks, vs + c, pl)
    np.testing.assert_allclose(o3, o + c, rtol=1e-12, atol=1e-12)


def test_ragged_prefix_padding_is_never_read():
    rng = np.random.default_rng(9)
    q, kp, vp, kb, vb, ks, vs = _rand(rng, 3, 2, 64, 4, 30, 5)
    pl = np.array([30, 17, 1])
    o = attend(q, kp, vp, kb, vb, ks, vs, pl)
    kp2, vp2 = kp.copy(), vp.copy()
    for b, P in enumerate(pl):
        kp2[b, :, P:] = 1e3 * rng.standard_normal(kp2[b, :, P:].shape)
        vp2[b, :, P:] = 1e3
    o2 = attend(q, kp2, vp2, kb, vb, ks, vs, pl)
    np.testing.assert_array_equal(o, o2)
    # and the live part is read: a shorter prefix changes the result
    o3 = attend(q, kp, vp, kb, vb, ks, vs, pl - np.array([1, 1, 0]))
    assert np.abs(o3[0] - o[0]).max() > 1e-6


def test_score_scale_is_inverse_sqrt_head_dim():
    # with one key aligned to q and one orthogonal, weights follow exp(|q|^2/sqrt(D))
    D = 64
    q = np.zeros((1, 1, 1, D)); q[..., 0] = 4.0
    kp = np.zeros((1, 1, 1, D)); kp[..., 0] = 4.0       # score 16/8 = 2
    kb = np.zeros((1, 1, 1, D)); kb[..., 1] = 4.0       # score 0
    vp = np.zeros((1, 1, 1, D)); vp[..., 2] = 1.0
    vb = np.zeros((1, 1, 1, D)); vb[..., 3] = 1.0
    z = np.zeros((1, 1, 0, D))
    o = attend(q, kp, vp, kb, vb, z, z, np.ones(1, int))
    w = math.exp(2.0) / (math.exp(2.0) + 1.0)
    assert abs(o[0, 0, 0, 2] - w) < 1e-14 and abs(o[0, 0, 0, 3] - (1 - w)) < 1e-14
