"""dblk_lmhead_confidence_commit_noalloc against dblk_lmhead_confidence_commit.

The allocation-free variant keeps its scratch in a per-GPU device array
instead of a caller workspace; its outputs must be bit-identical to the
workspace call's on every LM-head path (the fused row kernel, the K-outer
kernel, the GEMM with masked-row compaction).  Each case makes two calls in
a row on the shared scratch, the second with a smaller input, and a GEMM call
(which leaves softmax partials where the row kernels keep their arrival
counters) followed by row-kernel calls, so that each call must start clean
whatever the previous one left.  Compared bit for bit: tokens, mask,
n_committed, and conf / argmax of every row masked on entry.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_wise_decoding_amd import dblock
from synth import custom_workload, make_inputs
from tests.gpu_util import note, require_gpu, upload

pytestmark = pytest.mark.gpu


def _case(key, B, L, H, D, V):
    w = custom_workload(f"na{key}", 200 + key, B=B, H=H, D=D, L=L, P_cap=16, S=16, V=V,
                        mask_p=0.5)
    return w, make_inputs(w, parts=("lmhead", "commit"))


def _both(dev, w, inp):
    d = upload(inp, dev)
    B, L = w.B, w.L
    outs = []
    for noalloc in (False, True):
        conf = torch.full((B, L), -7.0, dtype=torch.float32, device=dev)
        amax = torch.full((B, L), -9, dtype=torch.int32, device=dev)
        tok, msk = d["tokens"].clone(), d["mask"].clone()
        n = torch.full((B,), -1, dtype=torch.int32, device=dev)
        if noalloc:
            dblock.dblk_lmhead_confidence_commit_noalloc(d["h"], d["w"], conf, amax, tok, msk,
                                                        w.tau, n)
        else:
            dblock.dblk_lmhead_confidence_commit(d["h"], d["w"], conf, amax, tok, msk, w.tau, n)
        torch.cuda.synchronize()
        outs.append((conf, amax, tok, msk, n))
    masked = d["mask"].bool()
    (c1, a1, t1, m1, n1), (c2, a2, t2, m2, n2) = outs
    for name, x, y in (("conf", c1[masked], c2[masked]), ("argmax", a1[masked], a2[masked]),
                       ("tokens", t1, t2), ("mask", m1, m2), ("n", n1, n2)):
        assert torch.equal(x, y), name
    assert int(n1.sum()) >= B


# (first call, second smaller call): fused row kernel (d = 2048, the LLaDA-MoE
# head), K-outer kernel (d = 320), GEMM path (B*L >= 256)
PAIRS = {
    "row-kernel": ((1, 1, 64, 16, 128, 157184), (2, 1, 32, 2, 128, 4096)),
    "k-outer": ((3, 2, 64, 5, 64, 7001), (4, 1, 16, 5, 64, 3000)),
    "gemm": ((5, 6, 64, 2, 128, 7000), (6, 4, 64, 2, 64, 5000)),
}


@pytest.mark.parametrize("path", list(PAIRS))
def test_noalloc_matches_workspace_call_twice(path):
    dev = require_gpu()
    for step, (key, B, L, H, D, V) in enumerate(PAIRS[path]):
        note(f"noalloc {path} call {step}: B={B} L={L} d={H * D} V={V}")
        w, inp = _case(key, B, L, H, D, V)
        _both(dev, w, inp)


def test_noalloc_after_another_plan():
    """A GEMM-path call leaves partials over the row kernel's counter slots;
    the row-kernel calls after it must still match."""
    dev = require_gpu()
    for key, B, L, H, D, V in ((7, 6, 64, 2, 128, 7000), (8, 1, 64, 16, 128, 40000),
                               (9, 1, 64, 16, 128, 40000)):
        note(f"noalloc plan switch: B={B} L={L} d={H * D} V={V}")
        w, inp = _case(key, B, L, H, D, V)
        _both(dev, w, inp)


def test_noalloc_rejects_oversize_before_running():
    dev = require_gpu()
    lib = dblock.load_library()
    B, L, d, V = 64, 64, 128, 157184          # GEMM partials 4096 x 614 x 16 B > the scratch
    assert dblock.lmhead_workspace_size(B * L, d, V) > dblock.NOALLOC_SCRATCH_BYTES
    h = torch.zeros(B * L, d, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(V, d, dtype=torch.bfloat16, device=dev)
    conf = torch.zeros(B, L, dtype=torch.float32, device=dev)
    amax = torch.zeros(B, L, dtype=torch.int32, device=dev)
    tok = torch.zeros(B, L, dtype=torch.int32, device=dev)
    msk = torch.ones(B, L, dtype=torch.uint8, device=dev)
    st = lib.dblk_lmhead_confidence_commit_noalloc(h.data_ptr(), W.data_ptr(), d, V,
                                                   conf.data_ptr(), amax.data_ptr(),
                                                   tok.data_ptr(), msk.data_ptr(), B, L, 0.9,
                                                   None, None)
    torch.cuda.synchronize()
    assert st == 4                             # DBLK_ERR_WORKSPACE
    assert bool((tok == 0).all()) and bool((msk == 1).all())   # nothing ran
