"""Pins for the oracle's LM head, confidence and argmax (CPU only).

Pinned by scipy's softmax/logsumexp, closed forms (one spike among equal
logits, exact ties), one-hot vocabulary matrices that expose the operand
orientation, sorting for the top-2 gap, and the planted-spike identity of the
input recipe (h = a W[t] / ||W[t]||^2 gives logit a at t).
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import confidence_from_logits, lm_logits, lmhead_confidence


def test_matches_scipy_softmax():
    rng = np.random.default_rng(11)
    l = rng.standard_normal((7, 300)) * 5
    conf, a, gap = confidence_from_logits(l)
    p = softmax(l, axis=1)
    np.testing.assert_allclose(conf, p.max(axis=1), rtol=1e-13)
    np.testing.assert_array_equal(a, p.argmax(axis=1))
    np.testing.assert_allclose(conf, np.exp(l.max(axis=1) - logsumexp(l, axis=1)), rtol=1e-13)


def test_single_spike_closed_form():
    for V, a, pos in [(4096, 7.5, 17), (157184, 24.0, 156895), (10, 0.0, 3)]:
        l = np.zeros((1, V)); l[0, pos] = a
        conf, amax, gap = confidence_from_logits(l)
        exp = math.exp(a) / (math.exp(a) + V - 1)
        assert abs(conf[0] - exp) < 1e-15 * max(1, exp) * 10
        if a > 0:
            assert amax[0] == pos and abs(gap[0] - a) < 1e-15
        else:
            assert amax[0] == 0 and gap[0] == 0.0     # all equal: lowest index wins, gap 0


def test_tie_goes_to_lowest_index():
    l = np.zeros((1, 50)); l[0, 31] = 3.0; l[0, 9] = 3.0
    conf, a, gap = confidence_from_logits(l)
    assert a[0] == 9 and gap[0] == 0.0
    assert abs(conf[0] - math.exp(3) / (2 * math.exp(3) + 48)) < 1e-15


def test_shift_invariance_and_range():
    rng = np.random.default_rng(12)
    l = rng.standard_normal((5, 1000)) * 3
    c1, a1, g1 = confidence_from_logits(l)
    c2, a2, g2 = confidence_from_logits(l + 123.25)
    np.testing.assert_allclose(c1, c2, rtol=1e-12)
    np.testing.assert_array_equal(a1, a2)
    assert (c1 > 0).all() and (c1 <= 1).all() and (c1 >= 1.0 / 1000).all()


def test_gap_matches_sorted_difference():
    rng = np.random.default_rng(13)
    l = rng.standard_normal((9, 777))
    _, _, gap = confidence_from_logits(l)
    s = np.sort(l, axis=1)
    np.testing.assert_array_equal(gap, s[:, -1] - s[:, -2])


def test_one_hot_vocabulary_exposes_orientation():
    # W = permutation of the identity (V = d): logits are h's entries permuted,
    # l[:, t] = h[:, perm[t]]; a transposed operand would apply perm^-1 instead.
    rng = np.random.default_rng(14)
    d = 64
    perm = rng.permutation(d)
    W = np.eye(d)[perm]
    h = rng.standard_normal((3, d))
    l = lm_logits(h, W)
    np.testing.assert_array_equal(l, h[:, perm])
    conf, a, _ = lmhead_confidence(h, W)
    np.testing.assert_allclose(conf, softmax(h, axis=1).max(axis=1), rtol=1e-13)
    np.testing.assert_array_equal(perm[a], h.argmax(axis=1))


def test_non_square_vocabulary():
    rng = np.random.default_rng(15)
    d, V = 32, 200
    W = np.zeros((V, d)); idx = rng.integers(0, d, V); W[np.arange(V), idx] = 1.0
    h = rng.standard_normal((4, d))
    np.testing.assert_array_equal(lm_logits(h, W), h[:, idx])


def test_planted_spike_logit():
    rng = np.random.default_rng(16)
    V, d = 300, 128
    W = rng.standard_normal((V, d)) / math.sqrt(d)
    t, a = 123, 17.25
    h = (a / (W[t] @ W[t]) * W[t])[None]
    l = lm_logits(h, W)
    assert abs(l[0, t] - a) < 1e-12


@pytest.mark.parametrize("chunk", [1, 3, 64])
def test_row_chunking_and_subsets_agree(chunk):
    rng = np.random.default_rng(17)
    h = rng.standard_normal((10, 32)); W = rng.standard_normal((90, 32))
    full = lmhead_confidence(h, W, chunk=64)
    part = lmhead_confidence(h, W, chunk=chunk)
    sub = lmhead_confidence(h, W, rows=np.array([7, 2]), chunk=chunk)
    # BLAS may round a one-row product differently from a block product
    for x, y in zip(full, part):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)
    for x, y in zip(full, sub):
        np.testing.assert_allclose(x[[7, 2]], y, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(full[1], part[1])


def test_bf16_bits_path_matches_decoded_path():
    # W given as bf16 bit patterns is decoded slice by slice; the logits must
    # equal those from the fully decoded float64 matrix (chunk edges included)
    from oracle import bf16_bits_to_f64
    from synth import f32_to_bf16_bits
    rng = np.random.default_rng(18)
    Wb = f32_to_bf16_bits(rng.standard_normal((103, 64)).astype(np.float32))
    h = rng.standard_normal((5, 64))
    # (BLAS may sum a 7-row slice in a different order than the whole matrix)
    np.testing.assert_allclose(lm_logits(h, Wb, vchunk=7), lm_logits(h, bf16_bits_to_f64(Wb)),
                               rtol=1e-13, atol=1e-13)
    full = lmhead_confidence(h, bf16_bits_to_f64(Wb))
    bits = lmhead_confidence(h, Wb)
    np.testing.assert_allclose(full[0], bits[0], rtol=1e-13)
    np.testing.assert_array_equal(full[1], bits[1])
