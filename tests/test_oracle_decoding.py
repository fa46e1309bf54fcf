"""Pins of the oracle's block loop, end-of-text rule and dual-cache advance.

The block loop is checked against a closed form derived independently of its
step-by-step code: with confidences fixed over the iterations, step 0
commits every masked position meeting the threshold (or, if none does, the
most confident one) and every later step commits the most confident position
left, so the commit order is a sort.  The end-of-text rule is checked on
hand-worked rows and on invariants; the cache advance against concatenation.
"""
import itertools

import numpy as np
import pytest

from oracle import (block_schedule_unambiguous, block_schedule_violations, cache_append,
                    decode_block, threshold_commit, threshold_commit_eos)


def closed_form_schedule(conf, mask, tau):
    """commit_iter from a sort: hits at 0, the rest by (-conf, position)."""
    B, L = conf.shape
    g = np.full((B, L), -1, dtype=np.int32)
    for b in range(B):
        idx = np.flatnonzero(mask[b])
        if idx.size == 0:
            continue
        hits = idx[conf[b, idx] >= tau]
        rest = idx[conf[b, idx] < tau]
        order = rest[np.lexsort((rest, -conf[b, rest]))]
        g[b, hits] = 0
        start = 1 if hits.size else 0
        g[b, order] = start + np.arange(order.size)
    return g


def random_case(rng, B, L, p=0.5, ties=False):
    conf = rng.random((B, L)).astype(np.float32)
    if ties:
        conf = np.round(conf * 8) / 8
    mask = (rng.random((B, L)) < p).astype(np.uint8)
    amax = rng.integers(0, 1000, (B, L)).astype(np.int32)
    tok = rng.integers(0, 1000, (B, L)).astype(np.int32)
    return conf, amax, tok, mask


@pytest.mark.parametrize("tau", [0.0, 0.3, 0.9, 1.0, 1.5])
@pytest.mark.parametrize("ties", [False, True])
def test_block_loop_matches_sort_closed_form(tau, ties):
    rng = np.random.default_rng(7)
    conf, amax, tok, mask = random_case(rng, 6, 48, ties=ties)
    t2, m2, g, n_it, fin = decode_block(conf, amax, tok, mask, np.float32(tau))
    expect = closed_form_schedule(conf, mask.astype(bool), np.float32(tau))
    assert np.array_equal(g, expect)
    assert not m2.any()
    m = mask.astype(bool)
    assert np.array_equal(t2[m], amax[m]) and np.array_equal(t2[~m], tok[~m])
    assert np.array_equal(n_it, np.where(m.any(1), expect.max(1) + 1, 0))
    assert not fin.any()


def test_block_loop_one_per_step_above_one():
    """tau > 1: exactly one commit per step, the block empties in |masked| steps."""
    rng = np.random.default_rng(3)
    conf, amax, tok, mask = random_case(rng, 4, 32, p=0.7)
    _, m2, g, n_it, _ = decode_block(conf, amax, tok, mask, np.float32(1.25))
    for b in range(4):
        k = int(mask[b].sum())
        assert n_it[b] == k
        assert sorted(g[b][g[b] >= 0].tolist()) == list(range(k))
    assert not m2.any()


def test_block_loop_exhaustive_small():
    rng = np.random.default_rng(11)
    L = 7
    for trial in range(4):
        conf = (rng.random((1, L)) if trial % 2 else np.round(rng.random((1, L)) * 4) / 4)
        conf = conf.astype(np.float32)
        amax = np.arange(L, dtype=np.int32)[None] + 100
        tok = np.zeros((1, L), dtype=np.int32)
        for bits in itertools.product([0, 1], repeat=L):
            mask = np.array([bits], dtype=np.uint8)
            for tau in (0.25, 0.6, 1.01):
                _, _, g, n_it, _ = decode_block(conf, amax, tok, mask, np.float32(tau))
                assert np.array_equal(g, closed_form_schedule(conf, mask.astype(bool), np.float32(tau)))


def test_block_loop_truncated():
    rng = np.random.default_rng(5)
    conf, amax, tok, mask = random_case(rng, 3, 40, p=0.8)
    full = closed_form_schedule(conf, mask.astype(bool), np.float32(0.9))
    t2, m2, g, n_it, _ = decode_block(conf, amax, tok, mask, np.float32(0.9), max_iters=4)
    assert np.array_equal(g, np.where(full < 4, full, -1))
    left = full >= 4
    assert np.array_equal(m2.astype(bool), left)
    assert np.array_equal(t2[left], tok[left])


def test_schedule_checker_accepts_oracle_and_catches_mistakes():
    rng = np.random.default_rng(9)
    conf, amax, tok, mask = random_case(rng, 4, 64)
    conf64 = conf.astype(np.float64)
    _, _, g, n_it, _ = decode_block(conf, amax, tok, mask, np.float32(0.9))
    assert block_schedule_violations(conf64, mask, 0.9, g, n_it) == []
    # two positions of one later step swapped with a neighbour step's: still a
    # valid schedule only if their confidences are within the band
    b = 0
    late = np.flatnonzero(g[b] >= 2)
    i, j = late[np.argsort(g[b, late])][:2]
    bad = g.copy()
    bad[b, i], bad[b, j] = g[b, j], g[b, i]
    if abs(conf64[b, i] - conf64[b, j]) >= 1e-3:
        assert block_schedule_violations(conf64, mask, 0.9, bad, n_it)
    bad = g.copy()
    bad[b, np.flatnonzero(mask[b] == 0)[0]] = 0          # an unmasked position committed
    assert block_schedule_violations(conf64, mask, 0.9, bad, n_it)
    bad = g.copy()
    bad[b, late[0]] = -1                                 # one never committed
    assert block_schedule_violations(conf64, mask, 0.9, bad, n_it)
    assert block_schedule_violations(conf64, mask, 0.9, g, n_it + 1)
    bad = g.copy()                                       # a sure hit left for later
    hit = np.flatnonzero((g[b] == 0) & (conf64[b] >= 0.9 + 1e-3))
    if hit.size:
        bad[b, hit[0]] = g[b].max() + 1
        assert block_schedule_violations(conf64, mask, 0.9, bad, n_it)


def test_schedule_ambiguity_flags():
    conf = np.array([[0.95, 0.5, 0.3, 0.1], [0.9004, 0.5, 0.3, 0.1], [0.95, 0.5, 0.5005, 0.1]])
    mask = np.ones((3, 4), dtype=np.uint8)
    assert block_schedule_unambiguous(conf, mask, 0.9).tolist() == [True, False, False]
    # a near-tie among sure hits changes nothing: both are committed at step 0
    conf2 = np.array([[0.95, 0.9504, 0.3, 0.1]])
    assert block_schedule_unambiguous(conf2, np.ones((1, 4)), 0.9).tolist() == [True]


# ------------------------------------------------------------------ end of text

EOS = 7


def test_eos_worked_rows():
    # row: positions 0..7; masked 1, 3, 5, 6; position 3 commits EOS (conf 0.95);
    # unmasked position 7 holds a non-EOS token and is never rewritten
    conf = np.array([[0.1, 0.2, 0.1, 0.95, 0.1, 0.3, 0.4, 0.1]], dtype=np.float32)
    amax = np.array([[9, 11, 9, EOS, 9, 12, 13, 9]], dtype=np.int32)
    tok = np.array([[5, 0, 6, 0, 8, 0, 0, 21]], dtype=np.int32)
    mask = np.array([[0, 1, 0, 1, 0, 1, 1, 0]], dtype=np.uint8)
    t, m, n, fb, fin = threshold_commit_eos(conf, amax, tok, mask, np.float32(0.9), EOS)
    assert t.tolist() == [[5, 0, 6, EOS, 8, EOS, EOS, 21]]
    assert m.tolist() == [[0, 1, 0, 0, 0, 0, 0, 0]]
    assert n.tolist() == [3] and fin.tolist() == [1] and not fb[0]

    # an EOS already in the row (unmasked, position 2) fills the masked tail
    # even though this step's own commit (position 1, by fallback) is before it
    tok = np.array([[5, 0, EOS, 0, 8, 0, 0, 21]], dtype=np.int32)
    mask = np.array([[0, 1, 0, 1, 0, 1, 1, 0]], dtype=np.uint8)
    conf = np.array([[0.1, 0.8, 0.1, 0.2, 0.1, 0.3, 0.4, 0.1]], dtype=np.float32)
    t, m, n, fb, fin = threshold_commit_eos(conf, amax, tok, mask, np.float32(0.9), EOS)
    assert t.tolist() == [[5, 11, EOS, EOS, 8, EOS, EOS, 21]]
    assert m.tolist() == [[0] * 8] and n.tolist() == [4] and fb[0] and fin.tolist() == [1]

    # a masked EOS argmax that is not committed does not end the text
    conf = np.array([[0.1, 0.95, 0.1, 0.5, 0.1, 0.3, 0.4, 0.1]], dtype=np.float32)
    tok = np.array([[5, 0, 6, 0, 8, 0, 0, 21]], dtype=np.int32)
    t, m, n, fb, fin = threshold_commit_eos(conf, amax, tok, mask, np.float32(0.9), EOS)
    assert t.tolist() == [[5, 11, 6, 0, 8, 0, 0, 21]] and fin.tolist() == [0] and n.tolist() == [1]


def test_eos_invariants_random():
    rng = np.random.default_rng(21)
    for trial in range(200):
        B, L = 3, int(rng.integers(1, 40))
        conf = rng.random((B, L)).astype(np.float32)
        amax = rng.integers(0, 12, (B, L)).astype(np.int32)
        tok = rng.integers(0, 12, (B, L)).astype(np.int32)
        mask = (rng.random((B, L)) < 0.6).astype(np.uint8)
        tau = np.float32(rng.choice([0.3, 0.9, 1.1]))
        t0, m0, n0, _ = threshold_commit(conf, amax, tok, mask, tau)
        t, m, n, _, fin = threshold_commit_eos(conf, amax, tok, mask, tau, EOS)
        for b in range(B):
            eos_pos = [i for i in range(L) if not m0[b, i] and t0[b, i] == EOS]
            assert fin[b] == (1 if eos_pos else 0)
            e = eos_pos[0] if eos_pos else L
            # up to and including e: exactly the plain step
            assert np.array_equal(t[b, :e + 1], t0[b, :e + 1])
            assert np.array_equal(m[b, :e + 1], m0[b, :e + 1])
            # after e: nothing masked; previously masked positions became EOS
            assert not m[b, e + 1:].any()
            filled = m0[b, e + 1:].astype(bool)
            assert (t[b, e + 1:][filled] == EOS).all()
            assert np.array_equal(t[b, e + 1:][~filled], t0[b, e + 1:][~filled])
            assert n[b] == n0[b] + filled.sum()
        # no EOS anywhere: identical to the plain step
    conf = rng.random((2, 16)).astype(np.float32)
    amax = rng.integers(100, 200, (2, 16)).astype(np.int32)
    tok = rng.integers(100, 200, (2, 16)).astype(np.int32)
    mask = np.ones((2, 16), dtype=np.uint8)
    a = threshold_commit(conf, amax, tok, mask, np.float32(0.5))
    b_ = threshold_commit_eos(conf, amax, tok, mask, np.float32(0.5), EOS)
    assert all(np.array_equal(x, y) for x, y in zip(a, b_[:4])) and not b_[4].any()


def test_block_loop_with_eos_ends_the_text():
    rng = np.random.default_rng(4)
    conf = rng.random((2, 24)).astype(np.float32)
    amax = rng.integers(100, 200, (2, 24)).astype(np.int32)
    amax[0, 10] = EOS
    conf[0, 10] = 0.99              # committed at step 0: everything masked after it is EOS
    tok = np.full((2, 24), 3, dtype=np.int32)
    mask = np.ones((2, 24), dtype=np.uint8)
    t, m, g, n_it, fin = decode_block(conf, amax, tok, mask, np.float32(0.9), eos_id=EOS)
    assert not m.any() and fin.tolist() == [1, 0]
    # after it: positions meeting the threshold in that same step keep their
    # argmax, the others are filled with EOS; all of them at step 0
    hit = conf[0, 11:] >= np.float32(0.9)
    assert np.array_equal(t[0, 11:], np.where(hit, amax[0, 11:], EOS)) and (g[0, 11:] == 0).all()
    assert np.array_equal(t[0, :10], amax[0, :10])
    # the text part (positions < 10) follows the plain loop's order
    _, _, g_plain, _, _ = decode_block(conf[:, :10], amax[:, :10], tok[:, :10], mask[:, :10],
                                       np.float32(0.9))
    assert np.array_equal(g[0, :10], g_plain[0])
    assert n_it[0] == g[0].max() + 1


# ------------------------------------------------------------------ cache advance

def test_cache_append_is_concatenation():
    rng = np.random.default_rng(2)
    B, H, P_cap, L, D = 4, 3, 40, 8, 16
    kp = rng.standard_normal((B, H, P_cap, D))
    vp = rng.standard_normal((B, H, P_cap, D))
    kb = rng.standard_normal((B, H, L, D))
    vb = rng.standard_normal((B, H, L, D))
    plen = np.array([0, 17, 33, -5], dtype=np.int32)      # 33 + 8 > 40: does not fit
    nk, nv, nl, app = cache_append(kp, vp, kb, vb, plen)
    assert nl.tolist() == [8, 25, 33, 8] and app.tolist() == [8, 8, 0, 8]
    for b in range(B):
        P_b = min(max(int(plen[b]), 0), P_cap)
        for h in range(H):
            if app[b]:
                want = np.concatenate([kp[b, h, :P_b], kb[b, h]])
                assert np.array_equal(nk[b, h, :P_b + L], want)
                assert np.array_equal(nv[b, h, :P_b + L], np.concatenate([vp[b, h, :P_b], vb[b, h]]))
                assert np.array_equal(nk[b, h, P_b + L:], kp[b, h, P_b + L:])
            else:
                assert np.array_equal(nk[b, h], kp[b, h]) and np.array_equal(nv[b, h], vp[b, h])
    assert not np.shares_memory(nk, kp)
