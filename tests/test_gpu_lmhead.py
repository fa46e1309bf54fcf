"""dblk_lmhead_confidence vs the fp64 oracle on sizes the oracle finishes in
seconds: several 16-row vocabulary tiles, ragged vocabulary tails, partial
64-row chunks of M, several chunks of M, and the GEMM path for M >= 256
(partial 256-row tiles in both dimensions).

Bar: confidence within 1e-3 absolute everywhere (observed errors are ~1e-6);
argmax identical wherever the oracle's top-2 logit gap is at least 1e-3.
"""
import numpy as np
import pytest
import torch

from block_wise_decoding_amd import dblock
from oracle import bf16_bits_to_f64, lmhead_confidence
from synth import custom_workload, make_inputs
from tests.gpu_util import bf16, note, require_gpu, run_lmhead

pytestmark = pytest.mark.gpu

CONF_TOL = 1e-3
GAP = 1e-3


def _compare(inp, dev, label):
    d = {"h": bf16(inp["h"], dev), "w": bf16(inp["w"], dev)}
    conf, amax = run_lmhead(d)
    torch.cuda.synchronize()
    conf = conf.cpu().numpy(); amax = amax.cpu().numpy()
    rc, ra, rg = lmhead_confidence(bf16_bits_to_f64(inp["h"]), inp["w"])
    err = np.abs(conf - rc).max()
    ok = rg >= GAP
    mism = int((amax[ok] != ra[ok]).sum())
    note(f"{label}: max|conf err|={err:.2e} argmax mismatches={mism} excluded(gap<1e-3)={int((~ok).sum())}")
    assert err < CONF_TOL
    assert mism == 0
    assert ((amax >= 0) & (amax < inp["w"].shape[0])).all()
    return conf, amax


@pytest.mark.parametrize("M,d,V", [
    (64, 256, 4096),      # one block of the tiny workload
    (32, 256, 4096),      # half an M chunk
    (1, 64, 17),          # one row, vocabulary smaller than a tile
    (64, 128, 5000),      # ragged vocabulary tail (5000 = 312 tiles + 8 rows)
    (65, 192, 3001),      # two M chunks, the second holding one row
    (130, 512, 20011),    # three M chunks, prime vocabulary
    (64, 2048, 40000),    # LLaDA-MoE hidden size, many workgroups
    (16, 4096, 12345),    # LLaDA-8B hidden size
    (96, 4096, 3000),     # K-outer kernel: two M chunks at d = 4096
    (200, 4096, 30000),   # K-outer kernel: four M chunks (the last of 8 rows), 7-8 tiles per workgroup
    (64, 320, 7001),      # K-outer kernel: five 64-k stages, 1-2 tiles per workgroup (idle waves)
    (64, 16384, 3000),    # the largest hidden size the library takes
    (8, 640, 140000),     # K-outer kernel: three passes per workgroup, the last nearly empty
    (8, 64, 400000),      # K-outer kernel: seven passes of one k stage each (every step ends a pass)
    (64, 256, 100),       # row kernel with 7 workgroups: fewer than 8 merge groups
    (64, 1024, 1000),     # staged row kernel, 63 workgroups in 8 uneven merge groups
    (128, 2048, 600),     # two M chunks of the staged row kernel, 38 workgroups
    # many block rows: the MFMA GEMM path (256 x 256 tiles, XCD super-tiles)
    (256, 256, 4096),     # one h tile, 16 vocabulary tiles
    (300, 512, 5000),     # partial h tile and partial vocabulary tile
    (513, 2048, 20011),   # three h tiles (one row in the last), prime vocabulary
    (1024, 128, 3000),    # two k stages, four h tiles
    (600, 4096, 9000),    # LLaDA-8B hidden size
    (256, 192, 3000),     # odd number of k stages (3)
    (260, 64, 1000),      # a single k stage
    (424, 256, 3000),     # last h tile: first half full (4 x 32 rows), second half 2 of its 32-row tiles
    (474, 512, 4001),     # last h tile: second half 3 of its 32-row tiles, the last one ragged
])
def test_lmhead_small(M, d, V):
    dev = require_gpu()
    note(f"lmhead M={M} d={d} V={V}")
    w = custom_workload(f"lm{M}_{d}_{V}", M + d + V, B=1, L=M, H=d // 64, D=64, V=V, a_max=24.0)
    inp = make_inputs(w, parts=("lmhead",))
    _compare(inp, dev, f"M={M} d={d} V={V}")


def test_ties_go_to_lowest_index_across_workgroups():
    # the same logit at many vocabulary rows spread over different workgroups:
    # identical W rows give bit-identical fp32 logits on every path
    dev = require_gpu()
    rng = np.random.default_rng(3)
    V, d, M = 50000, 256, 8
    Wf = (rng.standard_normal((V, d)) / 16).astype(np.float32)
    top = rng.standard_normal(d).astype(np.float32)
    rows = [49999, 31000, 20001, 777, 40000]
    Wf[rows] = top
    from synth import f32_to_bf16_bits
    Wb = f32_to_bf16_bits(Wf)
    hb = f32_to_bf16_bits((np.tile(top, (M, 1)) * 3).astype(np.float32))
    conf, amax = _compare({"h": hb, "w": Wb}, dev, "ties")
    assert (amax == min(rows)).all()


def test_deterministic_and_workspace_reuse():
    dev = require_gpu()
    w = custom_workload("lmdet", 77, B=1, L=64, H=4, D=64, V=30000)
    inp = make_inputs(w, parts=("lmhead",))
    h, W = bf16(inp["h"], dev), bf16(inp["w"], dev)
    ws = dblock.alloc_workspace(dblock.lmhead_workspace_size(64, 256, 30000), dev)
    outs = []
    for _ in range(4):      # the arrival counter must re-arm itself every call
        c = torch.empty(64, dtype=torch.float32, device=dev)
        a = torch.empty(64, dtype=torch.int32, device=dev)
        dblock.dblk_lmhead_confidence(h, W, c, a, workspace=ws)
        outs.append((c.cpu().numpy(), a.cpu().numpy()))
    assert int(ws[:4].view(torch.int32).item()) == 0
    for c, a in outs[1:]:
        np.testing.assert_array_equal(c, outs[0][0])
        np.testing.assert_array_equal(a, outs[0][1])
