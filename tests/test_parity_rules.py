"""The comparison rules (exclusion set, attention error metric) on planted cases."""
import numpy as np

from oracle import attention_row_rel_err, compare_commit, exclusion_set


def test_band_and_gap_exclusions():
    conf = np.array([[0.9004, 0.95, 0.5, 0.8985, 0.97]])
    gap = np.array([[1.0, 1.0, 1.0, 1.0, 0.0005]])
    mask = np.ones((1, 5), np.uint8)
    E = exclusion_set(conf, gap, mask, 0.9)
    np.testing.assert_array_equal(E, [[True, False, False, False, True]])


def test_fallback_near_tie_excludes_both():
    conf = np.array([[0.5, 0.7004, 0.2, 0.7]])
    gap = np.ones((1, 4))
    mask = np.array([[1, 1, 1, 1]])
    E = exclusion_set(conf, gap, mask, 0.9)
    np.testing.assert_array_equal(E, [[False, True, False, True]])
    # no near-tie when an unmasked position is the close one
    E2 = exclusion_set(conf, gap, np.array([[1, 1, 1, 0]]), 0.9)
    assert not E2.any()


def test_compare_counts_only_kept_positions():
    E = np.array([[False, True, False]])
    assert compare_commit([[1, 2, 3]], [[0, 1, 0]], [[1, 9, 3]], [[0, 0, 0]], E) == 0
    assert compare_commit([[1, 2, 4]], [[0, 1, 0]], [[1, 9, 3]], [[0, 0, 0]], E) == 1


def test_attention_metric_is_per_row_relative():
    ref = np.ones((1, 2, 1, 4)); ref[0, 1] *= 100
    gpu = ref.copy(); gpu[0, 0, 0, 0] += 0.01; gpu[0, 1, 0, 0] += 0.5
    assert abs(attention_row_rel_err(gpu, ref) - 0.01) < 1e-12
