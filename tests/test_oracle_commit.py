"""Pins for the oracle's threshold parallel decoder (CPU only).

The decoder of the README's usage section commits, in one iteration, every
still-masked position whose confidence meets the threshold, and at least the
single most confident one.  Pinned by special cases (tau = 1, tau = 0, empty
mask, confidence exactly at tau), a stable sort (repeated commits with an
unreachable threshold follow descending confidence), and an exhaustive sweep
of every mask on short rows checked against the defining properties.
"""
import itertools

import numpy as np

from oracle import threshold_commit


def _conf(rng, B, L):
    # distinct values in (0, 1) so that ties only appear where a test plants them
    return rng.permutation(B * L).reshape(B, L).astype(np.float64) / (B * L + 1) + 1e-3


def test_tau_one_commits_only_the_best_masked():
    rng = np.random.default_rng(21)
    conf = _conf(rng, 3, 16)
    amax = rng.integers(0, 1000, (3, 16))
    tok = np.full((3, 16), -1); mask = rng.random((3, 16)) < 0.6; mask[:, 0] = True
    t2, m2, n, fb = threshold_commit(conf, amax, tok, mask, 1.0)
    assert (n == 1).all() and fb.all()
    for b in range(3):
        idx = np.flatnonzero(mask[b])
        best = idx[np.argmax(conf[b, idx])]
        assert t2[b, best] == amax[b, best] and m2[b, best] == 0
        assert (m2[b].astype(bool) == (mask[b] & (np.arange(16) != best))).all()


def test_tau_zero_commits_every_masked():
    rng = np.random.default_rng(22)
    conf = _conf(rng, 2, 20); amax = rng.integers(0, 50, (2, 20))
    mask = rng.random((2, 20)) < 0.5; mask[:, 3] = True
    tok = rng.integers(100, 200, (2, 20))
    t2, m2, n, fb = threshold_commit(conf, amax, tok, mask, 0.0)
    assert not m2.any() and (n == mask.sum(1)).all() and not fb.any()
    np.testing.assert_array_equal(t2, np.where(mask, amax, tok))


def test_empty_mask_is_a_no_op():
    conf = np.full((2, 8), 0.99); amax = np.arange(16).reshape(2, 8)
    tok = np.arange(16).reshape(2, 8) + 100; mask = np.zeros((2, 8), bool)
    t2, m2, n, fb = threshold_commit(conf, amax, tok, mask, 0.5)
    np.testing.assert_array_equal(t2, tok); assert not m2.any() and (n == 0).all() and not fb.any()


def test_threshold_is_inclusive_and_unmasked_never_committed():
    conf = np.array([[0.9, 0.95, 0.5, 0.97]], dtype=np.float32)
    amax = np.array([[1, 2, 3, 4]]); tok = np.array([[7, 7, 7, 7]])
    mask = np.array([[1, 0, 1, 0]], np.uint8)
    t2, m2, n, fb = threshold_commit(conf, amax, tok, mask, np.float32(0.9))
    np.testing.assert_array_equal(t2, [[1, 7, 7, 7]])
    np.testing.assert_array_equal(m2, [[0, 0, 1, 0]])
    assert n[0] == 1 and not fb[0]


def test_fallback_ignores_unmasked_and_breaks_ties_low():
    conf = np.array([[0.3, 0.8, 0.4, 0.4, 0.1]])
    amax = np.array([[10, 11, 12, 13, 14]]); tok = np.zeros((1, 5), int)
    mask = np.array([[1, 0, 1, 1, 1]])
    t2, m2, n, fb = threshold_commit(conf, amax, tok, mask, 0.9)
    assert fb[0] and n[0] == 1 and t2[0, 2] == 12 and m2[0, 2] == 0 and m2[0, 3] == 1


def test_repeated_unreachable_threshold_follows_descending_confidence():
    rng = np.random.default_rng(23)
    L = 24
    conf = _conf(rng, 1, L); amax = rng.integers(0, 9, (1, L))
    mask = rng.random((1, L)) < 0.7; mask[0, 5] = True
    order = [i for i in np.argsort(-conf[0], kind="stable") if mask[0, i]]
    tok = np.full((1, L), -1); m = mask.astype(np.uint8)
    seen = []
    for _ in range(int(mask.sum())):
        before = m.copy()
        tok, m, n, fb = threshold_commit(conf, amax, tok, m, 2.0)
        assert n[0] == 1
        seen.append(int(np.flatnonzero(before[0] & ~m[0].astype(bool))[0]))
    assert seen == order and not m.any()
    tok, m, n, fb = threshold_commit(conf, amax, tok, m, 2.0)
    assert n[0] == 0


def test_exhaustive_small_rows_satisfy_definition():
    rng = np.random.default_rng(24)
    L = 7
    for trial in range(6):
        conf = rng.random((1, L))
        amax = rng.integers(0, 99, (1, L)); tok = rng.integers(100, 199, (1, L))
        for tau in (0.0, 0.3, 0.6, 0.95, 1.0):
            for bits in itertools.product([0, 1], repeat=L):
                mask = np.array([bits], np.uint8)
                t2, m2, n, fb = threshold_commit(conf, amax, tok, mask, tau)
                C = mask[0].astype(bool) & ~m2[0].astype(bool)
                M = mask[0].astype(bool)
                assert not (m2[0].astype(bool) & ~M).any()            # C within the masked set
                assert (t2[0][~C] == tok[0][~C]).all()                  # others untouched
                assert (t2[0][C] == amax[0][C]).all()
                assert n[0] == C.sum()
                thr = M & (conf[0] >= tau)
                if thr.any():
                    assert (C == thr).all()
                elif M.any():
                    assert C.sum() == 1 and conf[0][C][0] == conf[0][M].max()
                else:
                    assert not C.any()


def test_higher_threshold_commits_a_subset():
    rng = np.random.default_rng(25)
    conf = rng.random((4, 32)); amax = rng.integers(0, 9, (4, 32))
    mask = rng.random((4, 32)) < 0.5; mask[:, 0] = True
    tok = np.zeros((4, 32), int)
    prev = None
    for tau in (0.2, 0.4, 0.6, 0.8):
        _, m2, _, fb = threshold_commit(conf, amax, tok, mask, tau)
        C = mask & ~m2.astype(bool)
        if prev is not None:
            ok = ~fb
            assert not (C[ok] & ~prev[ok]).any()
        prev = C
