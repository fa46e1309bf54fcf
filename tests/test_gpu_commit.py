"""dblk_threshold_commit vs the oracle's threshold decoder, bit for bit.

Both sides get the same float32 confidences and compare them with the same
float32 threshold, so every decision is taken in the same precision and the
results must be identical (no exclusion band here).
"""
import numpy as np
import pytest
import torch

from block_wise_decoding_amd import dblock
from oracle import threshold_commit
from tests.gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu


def _run(conf, amax, tok, mask, tau, dev):
    B, L = conf.shape
    c = torch.from_numpy(conf.astype(np.float32)).to(dev)
    a = torch.from_numpy(amax.astype(np.int32)).to(dev)
    t = torch.from_numpy(tok.astype(np.int32)).to(dev)
    m = torch.from_numpy(mask.astype(np.uint8)).to(dev)
    n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    dblock.dblk_threshold_commit(c, a, t, m, tau, n)
    torch.cuda.synchronize()
    return t.cpu().numpy(), m.cpu().numpy(), n.cpu().numpy()


def _check(conf, amax, tok, mask, tau, dev):
    c32 = conf.astype(np.float32)
    rt, rm, rn, _ = threshold_commit(c32, amax, tok, mask, np.float32(tau))
    gt, gm, gn = _run(c32, amax, tok, mask, tau, dev)
    np.testing.assert_array_equal(gt, rt)
    np.testing.assert_array_equal(gm.astype(bool), rm.astype(bool))
    np.testing.assert_array_equal(gn, rn)


@pytest.mark.parametrize("B,L", [(1, 1), (1, 16), (3, 64), (32, 128), (5, 333), (2, 4096)])
@pytest.mark.parametrize("tau", [0.0, 0.7, 0.9, 0.95, 1.0, 1.5])
def test_random_confidences(B, L, tau):
    dev = require_gpu()
    note(f"commit B={B} L={L} tau={tau}")
    rng = np.random.default_rng(B * 1000 + L)
    conf = rng.random((B, L)) ** 0.3
    amax = rng.integers(0, 157184, (B, L))
    mask = (rng.random((B, L)) < 0.5).astype(np.uint8)
    mask[0] = 0                                   # a row with nothing masked: no-op
    tok = np.where(mask == 1, 156895, rng.integers(0, 157184, (B, L)))
    _check(conf, amax, tok, mask, tau, dev)


def test_ties_exact_threshold_and_full_mask():
    dev = require_gpu()
    L = 200
    conf = np.full((4, L), 0.25, np.float32)
    conf[0, [150, 7, 99]] = 0.5          # fallback tie: lowest position (7) must win
    conf[1, [3, 4]] = np.float32(0.9)    # exactly at the threshold: committed
    conf[2, :] = 0.1                     # all equal, all masked: position 0
    amax = np.arange(4 * L).reshape(4, L)
    mask = np.ones((4, L), np.uint8)
    mask[3, :] = 0
    mask[3, 177] = 1
    tok = np.full((4, L), -1)
    _check(conf, amax, tok, mask, 0.9, dev)


def test_repeated_commits_drain_the_mask():
    dev = require_gpu()
    rng = np.random.default_rng(5)
    B, L = 3, 64
    conf = rng.random((B, L)).astype(np.float32)
    amax = rng.integers(0, 1000, (B, L))
    mask = np.ones((B, L), np.uint8)
    tok = np.full((B, L), -1)
    c = torch.from_numpy(conf).to(dev); a = torch.from_numpy(amax.astype(np.int32)).to(dev)
    t = torch.from_numpy(tok.astype(np.int32)).to(dev); m = torch.from_numpy(mask).to(dev)
    rt, rm = tok.copy(), mask.copy()
    for it in range(L):
        dblock.dblk_threshold_commit(c, a, t, m, 2.0)        # unreachable: one per call
        rt, rm, _, _ = threshold_commit(conf, amax, rt, rm, np.float32(2.0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t.cpu().numpy(), rt)
    assert not m.cpu().numpy().any() and not rm.any()
