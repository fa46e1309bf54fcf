"""GPU parity of what surrounds one iteration: the decoder step with end-of-text
handling, the device-side block loop, the dual-cache advance and suffix
windows, all called through the C ABI and compared with the fp64 oracle.

Bars: integer outputs (tokens, mask, commit iterations, counts, flags, cache
bytes) bit-exact where the oracle's decisions are unambiguous; elsewhere the
block loop's schedule must be a valid run of the decoder on confidences
within 1e-3 of the oracle's (oracle.block_schedule_violations); confidence
within 1e-3; attention per-row relative error within 1e-2.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_wise_decoding_amd import dblock
from oracle import (attend, attention_row_rel_err, bf16_bits_to_f64, block_schedule_unambiguous,
                    block_schedule_violations, cache_append, decode_block, lmhead_confidence,
                    threshold_commit_eos)
from synth import WORKLOADS, make_inputs
from synth.workloads import custom_workload
from tests.gpu_util import bf16, bf16_to_np, note, require_gpu, upload

pytestmark = pytest.mark.gpu

BAND = 1e-3


# ------------------------------------------------------------------ decoder step + EOS

@pytest.mark.parametrize("B,L", [(1, 16), (4, 64), (3, 128), (2, 1000), (1, 4096), (64, 32)])
def test_commit_eos_matches_oracle(B, L):
    dev = require_gpu()
    note(f"commit_eos B={B} L={L}")
    rng = np.random.default_rng(1000 * B + L)
    eos = 7
    conf = rng.random((B, L)).astype(np.float32)
    amax = rng.integers(0, 40, (B, L)).astype(np.int32)      # EOS is one of 40 ids
    tok = rng.integers(0, 40, (B, L)).astype(np.int32)
    mask = (rng.random((B, L)) < 0.5).astype(np.uint8)
    g_tok = torch.from_numpy(tok).to(dev)
    g_msk = torch.from_numpy(mask).to(dev)
    g_conf = torch.from_numpy(conf).to(dev)
    g_amax = torch.from_numpy(amax).to(dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    fin = torch.empty(B, dtype=torch.uint8, device=dev)
    r_tok, r_msk = tok, mask
    for step, tau in enumerate((0.9, 0.95, 0.5)):            # the state evolves over steps
        dblock.dblk_threshold_commit_eos(g_conf, g_amax, g_tok, g_msk, tau, eos, n, fin)
        r_tok, r_msk, r_n, _, r_fin = threshold_commit_eos(conf, amax, r_tok, r_msk,
                                                           np.float32(tau), eos)
        torch.cuda.synchronize()
        assert np.array_equal(g_tok.cpu().numpy(), r_tok), f"tokens, step {step}"
        assert np.array_equal(g_msk.cpu().numpy(), r_msk), f"mask, step {step}"
        assert np.array_equal(n.cpu().numpy(), r_n), f"n_committed, step {step}"
        assert np.array_equal(fin.cpu().numpy(), r_fin), f"finished, step {step}"


@pytest.mark.parametrize("B,L,H,D,V", [(1, 64, 16, 128, 157184), (4, 16, 4, 128, 5000),
                                       (2, 32, 2, 128, 3000), (1, 128, 4, 128, 4000),
                                       (3, 64, 32, 128, 9000), (8, 64, 2, 128, 3000),
                                       (16, 4, 4, 64, 2000)])
def test_lmhead_commit_fused_matches_two_calls(B, L, H, D, V):
    """dblk_lmhead_confidence_commit == dblk_lmhead_confidence + dblk_threshold_commit,
    bit for bit, over three consecutive steps (fused for L <= 64 with fewer
    than 256 rows; two launches for L = 128 and on the GEMM path)."""
    dev = require_gpu()
    w = custom_workload(f"lmc{B}x{L}", 37, B=B, H=H, D=D, L=L, P_cap=32, S=16, V=V, mask_p=0.7)
    note(f"lmhead_commit fused B={B} L={L} d={w.d} V={V}")
    inp = make_inputs(w, parts=("lmhead", "commit"))
    d = upload(inp, dev)
    t1, m1 = d["tokens"].clone(), d["mask"].clone()
    t2, m2 = d["tokens"].clone(), d["mask"].clone()
    c1 = torch.empty(B, L, dtype=torch.float32, device=dev)
    a1 = torch.empty(B, L, dtype=torch.int32, device=dev)
    c2, a2 = torch.empty_like(c1), torch.empty_like(a1)
    n1 = torch.empty(B, dtype=torch.int32, device=dev)
    n2 = torch.empty_like(n1)
    for step, tau in enumerate((w.tau, w.tau, 0.5)):
        masked = m1.bool().clone()            # conf/argmax are promised on these rows
        dblock.dblk_lmhead_confidence(d["h"], d["w"], c1.view(-1), a1.view(-1))
        dblock.dblk_threshold_commit(c1, a1, t1, m1, tau, n1)
        dblock.dblk_lmhead_confidence_commit(d["h"], d["w"], c2, a2, t2, m2, tau, n2)
        torch.cuda.synchronize()
        for name, x, y in (("conf", c1[masked], c2[masked]), ("argmax", a1[masked], a2[masked]),
                           ("tokens", t1, t2), ("mask", m1, m2), ("n", n1, n2)):
            assert torch.equal(x, y), f"{name}, step {step}"
    assert int(n1.sum()) > 0


@pytest.mark.parametrize("p_mask", [0.0, 0.03, 0.5, 1.0])
def test_lmhead_commit_masked_row_compaction(p_mask):
    """GEMM path (B*L >= 256): only masked rows go through the LM head.  Their
    conf/argmax equal the dense LM head's bit for bit, the other rows keep
    what was there, and the commit equals the two-call path."""
    dev = require_gpu()
    B, L = 6, 64
    w = custom_workload("cmp", 38, B=B, H=2, D=128, L=L, P_cap=32, S=16, V=7000, mask_p=0.5)
    note(f"masked-row compaction B={B} L={L} p={p_mask}")
    inp = make_inputs(w, parts=("lmhead", "commit"))
    rng = np.random.default_rng(int(p_mask * 100) + 1)
    inp["mask"] = (rng.random((B, L)) < p_mask).astype(np.uint8)
    d = upload(inp, dev)
    c1 = torch.empty(B, L, dtype=torch.float32, device=dev)
    a1 = torch.empty(B, L, dtype=torch.int32, device=dev)
    t1, m1 = d["tokens"].clone(), d["mask"].clone()
    dblock.dblk_lmhead_confidence(d["h"], d["w"], c1.view(-1), a1.view(-1))
    dblock.dblk_threshold_commit(c1, a1, t1, m1, w.tau)
    c2 = torch.full((B, L), -7.0, dtype=torch.float32, device=dev)
    a2 = torch.full((B, L), -9, dtype=torch.int32, device=dev)
    t2, m2 = d["tokens"].clone(), d["mask"].clone()
    dblock.dblk_lmhead_confidence_commit(d["h"], d["w"], c2, a2, t2, m2, w.tau)
    torch.cuda.synchronize()
    masked = torch.from_numpy(inp["mask"].astype(bool)).to(dev)
    assert torch.equal(c2[masked], c1[masked]) and torch.equal(a2[masked], a1[masked])
    assert bool((c2[~masked] == -7.0).all()) and bool((a2[~masked] == -9).all())
    assert torch.equal(t1, t2) and torch.equal(m1, m2)


@pytest.mark.parametrize("p_mask", [0.0, 0.03, 0.5, 1.0])
@pytest.mark.parametrize("B,L,H,D,V", [(1, 64, 16, 128, 7000), (2, 32, 8, 128, 5000),
                                       (1, 64, 4, 128, 3000), (4, 16, 2, 128, 3000),
                                       (1, 16, 16, 128, 4000), (3, 64, 8, 128, 3000),
                                       (1, 48, 16, 128, 3000)])
def test_lmhead_commit_masked_row_compaction_rows(B, L, H, D, V, p_mask):
    """Rows-outer LM head (B*L < 256, d = 256..2048): only the masked rows of
    each 64-row chunk go through the head.  Their conf/argmax equal the dense
    LM head's bit for bit, the other rows keep what was there, and the commit
    equals the two-call path (fused for L a power of two, else two launches)."""
    dev = require_gpu()
    w = custom_workload(f"cr{B}x{L}", 39, B=B, H=H, D=D, L=L, P_cap=32, S=16, V=V, mask_p=0.5)
    note(f"row-kernel compaction B={B} L={L} d={w.d} V={V} p={p_mask}")
    inp = make_inputs(w, parts=("lmhead", "commit"))
    rng = np.random.default_rng(int(p_mask * 100) + 7 * B + L)
    inp["mask"] = (rng.random((B, L)) < p_mask).astype(np.uint8)
    d = upload(inp, dev)
    c1 = torch.empty(B, L, dtype=torch.float32, device=dev)
    a1 = torch.empty(B, L, dtype=torch.int32, device=dev)
    t1, m1 = d["tokens"].clone(), d["mask"].clone()
    dblock.dblk_lmhead_confidence(d["h"], d["w"], c1.view(-1), a1.view(-1))
    dblock.dblk_threshold_commit(c1, a1, t1, m1, w.tau)
    c2 = torch.full((B, L), -7.0, dtype=torch.float32, device=dev)
    a2 = torch.full((B, L), -9, dtype=torch.int32, device=dev)
    t2, m2 = d["tokens"].clone(), d["mask"].clone()
    dblock.dblk_lmhead_confidence_commit(d["h"], d["w"], c2, a2, t2, m2, w.tau)
    torch.cuda.synchronize()
    masked = torch.from_numpy(inp["mask"].astype(bool)).to(dev)
    assert torch.equal(c2[masked], c1[masked]) and torch.equal(a2[masked], a1[masked])
    assert bool((c2[~masked] == -7.0).all()) and bool((a2[~masked] == -9).all())
    assert torch.equal(t1, t2) and torch.equal(m1, m2)


# ------------------------------------------------------------------ block loop

def _decode_gpu(d, w, tau, eos_id=-1, max_iters=0, sentinel=False):
    dev = d["h"].device
    B, L = w.B, w.L
    out = torch.empty_like(d["q"])
    conf = torch.empty(B, L, dtype=torch.float32, device=dev)
    amax = torch.empty(B, L, dtype=torch.int32, device=dev)
    if sentinel:
        out.fill_(-3.0)
        conf.fill_(-1.0)
        amax.fill_(-5)
    tok = d["tokens"].clone()
    msk = d["mask"].clone()
    citer = torch.empty(B, L, dtype=torch.int32, device=dev)
    nit = torch.empty(B, dtype=torch.int32, device=dev)
    fin = torch.zeros(B, dtype=torch.uint8, device=dev)
    args = dblock.decode_args(d["q"], d["kp"], d["vp"], d["kb"], d["vb"], d["ks"], d["vs"],
                              d["prefix_len"], out, d["h"], d["w"], conf, amax, tok, msk, tau,
                              eos_id=eos_id, max_iters=max_iters, commit_iter=citer, n_iters=nit,
                              finished=fin)
    dblock.dblk_decode_block(args, device=dev)
    torch.cuda.synchronize()
    return {"o": bf16_to_np(out), "conf": conf.cpu().numpy(), "argmax": amax.cpu().numpy(),
            "tokens": tok.cpu().numpy(), "mask": msk.cpu().numpy(),
            "commit_iter": citer.cpu().numpy(), "n_iters": nit.cpu().numpy(),
            "finished": fin.cpu().numpy()}


def _oracle_conf(w, inp, seqs):
    rows = np.concatenate([np.arange(b * w.L, (b + 1) * w.L) for b in seqs])
    c, a, g = lmhead_confidence(bf16_bits_to_f64(inp["h"]), inp["w"], rows=rows)
    k = len(seqs)
    return c.reshape(k, w.L), a.reshape(k, w.L), g.reshape(k, w.L)


def _check_loop(w, inp, g, seqs):
    """Schedule validity, exactness where unambiguous, tokens, conf for the given sequences."""
    rc, ra, rgap = _oracle_conf(w, inp, seqs)
    m0 = inp["mask"][seqs].astype(bool)
    tok0 = inp["tokens"][seqs]
    gi, gn = g["commit_iter"][seqs], g["n_iters"][seqs]
    errs = block_schedule_violations(rc, m0, w.tau, gi, gn, BAND)
    assert errs == [], errs[:5]
    _, _, r_iter, r_n, _ = decode_block(rc.astype(np.float32), ra, tok0, m0, np.float32(w.tau))
    unamb = block_schedule_unambiguous(rc, m0, w.tau, BAND)
    for j in range(len(seqs)):
        if unamb[j]:
            assert np.array_equal(gi[j], r_iter[j]), f"sequence {seqs[j]}: schedule"
            assert gn[j] == r_n[j]
    diff = int((gi != r_iter).sum())
    assert not g["mask"][seqs].any(), "the block loop left masked positions"
    gt = g["tokens"][seqs]
    assert np.array_equal(gt[~m0], tok0[~m0]), "unmasked tokens changed"
    sure = m0 & (rgap >= BAND)
    assert np.array_equal(gt[sure], ra[sure]), "committed token != oracle argmax"
    # conf / argmax are promised on the positions masked at the start
    cerr = float(np.abs(g["conf"][seqs][m0] - rc[m0]).max()) if m0.any() else 0.0
    assert cerr <= 1e-3, cerr
    okg = (rgap >= BAND) & m0
    assert np.array_equal(g["argmax"][seqs][okg], ra[okg])
    note(f"  sequences {list(seqs)}: iterations {gn.tolist()}, ambiguous rows "
         f"{int((~unamb).sum())}, positions off the oracle's exact schedule {diff}, conf err {cerr:.2e}")
    return rc


LOOP_CASES = {
    "c0": lambda: WORKLOADS["c0"],
    # 4 x 64 = 256 block rows: the MFMA GEMM LM head with its per-tile skip
    "b4-gemm": lambda: custom_workload("b4-gemm", 31, B=4, H=4, D=64, L=64, P_cap=128, S=64,
                                       V=5000, mask_p=0.6),
    # 2 x 64 rows: two 64-row chunks of the row kernel, one per sequence
    "b2-rows": lambda: custom_workload("b2-rows", 32, B=2, H=4, D=128, L=64, P_cap=96, S=32,
                                       V=7000, mask_p=0.4),
    "c2-blk8": lambda: WORKLOADS["c2-blk8"],
}


@pytest.mark.parametrize("name", list(LOOP_CASES))
def test_decode_block_matches_oracle(name):
    dev = require_gpu()
    w = LOOP_CASES[name]()
    note(f"decode_block {name}: B={w.B} H={w.H} D={w.D} L={w.L} P_cap={w.P_cap} S={w.S} "
         f"V={w.V} d={w.d} tau={w.tau}")
    inp = make_inputs(w)
    g = _decode_gpu(upload(inp, dev), w, w.tau)
    _check_loop(w, inp, g, list(range(w.B)))
    # the attention output of the last iteration is the iteration's attention
    hs = range(w.H) if w.B * w.H <= 16 else (0, w.H - 1)
    for b in range(w.B):
        for h in hs:
            sl = lambda k: bf16_bits_to_f64(inp[k][b:b + 1, h:h + 1])
            ref = attend(bf16_bits_to_f64(inp["q"][b:b + 1, :, h:h + 1]), sl("kp"), sl("vp"),
                         sl("kb"), sl("vb"), sl("ks"), sl("vs"), inp["prefix_len"][b:b + 1])
            assert attention_row_rel_err(g["o"][b:b + 1, :, h:h + 1], ref) <= 1e-2


@pytest.mark.slow
def test_decode_block_throughput_workload_sampled():
    """B = 32, L = 128 (4096 rows, GEMM path); two sequences checked in full."""
    dev = require_gpu()
    w = WORKLOADS["c4-tau90"]
    note(f"decode_block c4-tau90: B={w.B} L={w.L} V={w.V} d={w.d}")
    inp = make_inputs(w)
    g = _decode_gpu(upload(inp, dev), w, w.tau)
    assert not g["mask"].any()
    _check_loop(w, inp, g, [0, w.B - 1])


def test_decode_block_skips_complete_sequences():
    """Sequences with nothing masked are skipped by every kernel of the loop:
    their attention output, confidences and argmax keep what was there."""
    dev = require_gpu()
    for name, done in (("b2-rows", [0]), ("b8-gemm", [0, 1, 2, 3]), ("b2-all", [0, 1])):
        if name == "b8-gemm":
            w = custom_workload(name, 33, B=8, H=2, D=64, L=64, P_cap=64, S=32, V=3000)
        else:
            w = custom_workload(name, 34, B=2, H=4, D=128, L=64, P_cap=96, S=32, V=7000)
        note(f"decode_block skip {name}: complete sequences {done}")
        inp = make_inputs(w)
        inp["mask"][done] = 0
        g = _decode_gpu(upload(inp, dev), w, w.tau, sentinel=True)
        for b in done:
            assert (g["conf"][b] == -1.0).all() and (g["argmax"][b] == -5).all(), b
            assert (g["o"][b] == -3.0).all(), b
            assert g["n_iters"][b] == 0 and (g["commit_iter"][b] == -1).all()
            assert np.array_equal(g["tokens"][b], inp["tokens"][b])
        live = [b for b in range(w.B) if b not in done]
        if live:
            _check_loop(w, inp, g, live)


def test_decode_block_truncated_iterations():
    dev = require_gpu()
    w = WORKLOADS["c0"]
    note("decode_block c0 max_iters=3")
    inp = make_inputs(w)
    d = upload(inp, dev)
    g = _decode_gpu(d, w, w.tau, max_iters=3)
    full = _decode_gpu(d, w, w.tau)
    # the first three steps are those of the complete run
    early = full["commit_iter"] < 3
    assert np.array_equal(g["commit_iter"], np.where(early, full["commit_iter"], -1))
    assert np.array_equal(g["mask"].astype(bool), inp["mask"].astype(bool) & ~early)
    assert np.array_equal(g["tokens"], np.where(early, full["tokens"], inp["tokens"]))


def _eos_case():
    """A small batch whose every decision is unambiguous, with an end of text
    in the middle of sequence 0.

    All positions are generated masked; the oracle's confidences then choose
    which stay masked: positions with a clear top-2 gap, confidence away from
    the threshold, and, below the threshold, confidences at least 2*band apart
    (so the fallback order cannot flip).  The EOS id is the argmax of a
    confident position in the middle of sequence 0, committed at step 0; the
    masked positions after it are then filled with EOS."""
    for key in range(40, 60):
        w = custom_workload(f"eos{key}", key, B=2, H=4, D=64, L=32, P_cap=64, S=32, V=4096,
                            mask_p=1.0, a_max=24.0)
        inp = make_inputs(w)
        rc, ra, rgap = _oracle_conf(w, inp, [0, 1])
        keep = np.zeros((2, w.L), dtype=bool)
        for b in range(2):
            low = []
            for i in np.argsort(-rc[b], kind="stable"):
                if rgap[b, i] < BAND or abs(rc[b, i] - w.tau) < BAND:
                    continue
                if rc[b, i] < w.tau and any(abs(rc[b, i] - c) < 2 * BAND for c in low):
                    continue
                keep[b, i] = True
                if rc[b, i] < w.tau:
                    low.append(rc[b, i])
        cand = [i for i in range(8, 24) if keep[0, i] and rc[0, i] >= w.tau + BAND]
        if not cand:
            continue
        c = cand[0]
        eos = int(ra[0, c])
        # the EOS id appears nowhere else among the masked positions' argmaxes
        if eos == w.mask_id or (ra[1][keep[1]] == eos).any() or (ra[0, :c][keep[0, :c]] == eos).any():
            continue
        if not keep[0, :c].any() or not keep[0, c + 1:].any():
            continue
        inp["mask"] = keep.astype(np.uint8)
        assert block_schedule_unambiguous(rc, keep, w.tau, BAND).all()
        return w, inp, eos, rc, ra
    pytest.fail("no EOS case among the candidate seeds")


def test_decode_block_eos_matches_oracle():
    dev = require_gpu()
    w, inp, eos, rc, ra = _eos_case()
    note(f"decode_block eos {w.name}: eos_id={eos}")
    g = _decode_gpu(upload(inp, dev), w, w.tau, eos_id=eos)
    r_tok, r_msk, r_iter, r_n, r_fin = decode_block(rc.astype(np.float32), ra, inp["tokens"],
                                                    inp["mask"], np.float32(w.tau), eos_id=eos)
    assert r_fin[0] == 1
    assert np.array_equal(g["tokens"], r_tok)
    assert np.array_equal(g["mask"], r_msk)
    assert np.array_equal(g["commit_iter"], r_iter)
    assert np.array_equal(g["n_iters"], r_n)
    assert np.array_equal(g["finished"], r_fin)


@pytest.mark.parametrize("name,chunk", [("c0", 1), ("c0", 5), ("b4-gemm", 3), ("c2-blk8", 4),
                                        ("c2-blk8", 64)])
def test_decode_block_run_matches_device_loop(name, chunk):
    """The pipelined driver gives the same block as the fully enqueued loop,
    and stops enqueuing within two chunks of the block's completion."""
    dev = require_gpu()
    w = LOOP_CASES[name]()
    note(f"decode_block_run {name} chunk={chunk}")
    inp = make_inputs(w)
    d = upload(inp, dev)
    ref = _decode_gpu(d, w, w.tau)
    B, L = w.B, w.L
    out = torch.empty_like(d["q"])
    conf = torch.empty(B, L, dtype=torch.float32, device=dev)
    amax = torch.empty(B, L, dtype=torch.int32, device=dev)
    tok = d["tokens"].clone()
    msk = d["mask"].clone()
    citer = torch.empty(B, L, dtype=torch.int32, device=dev)
    nit = torch.empty(B, dtype=torch.int32, device=dev)
    args = dblock.decode_args(d["q"], d["kp"], d["vp"], d["kb"], d["vb"], d["ks"], d["vs"],
                              d["prefix_len"], out, d["h"], d["w"], conf, amax, tok, msk, w.tau,
                              commit_iter=citer, n_iters=nit)
    n_enq = dblock.dblk_decode_block_run(args, chunk, device=dev)
    torch.cuda.synchronize()
    assert np.array_equal(tok.cpu().numpy(), ref["tokens"])
    assert not msk.cpu().numpy().any()
    assert np.array_equal(citer.cpu().numpy(), ref["commit_iter"])
    assert np.array_equal(nit.cpu().numpy(), ref["n_iters"])
    m0 = inp["mask"].astype(bool)
    assert np.array_equal(conf.cpu().numpy()[m0], ref["conf"][m0])
    need = int(ref["n_iters"].max())
    assert need <= n_enq <= min(L, (need // chunk + 2) * chunk), (need, n_enq)


def test_decode_block_graph_replay():
    """The loop captured into a HIP graph and replayed gives the eager result,
    replay after replay, with eager work in between."""
    dev = require_gpu()
    w = WORKLOADS["c0"]
    note("decode_block c0 graph capture")
    inp = make_inputs(w)
    d = upload(inp, dev)
    eager = _decode_gpu(d, w, w.tau)
    B, L = w.B, w.L
    out = torch.empty_like(d["q"])
    conf = torch.empty(B, L, dtype=torch.float32, device=dev)
    amax = torch.empty(B, L, dtype=torch.int32, device=dev)
    tok = d["tokens"].clone()
    msk = d["mask"].clone()
    citer = torch.empty(B, L, dtype=torch.int32, device=dev)
    nit = torch.empty(B, dtype=torch.int32, device=dev)
    args = dblock.decode_args(d["q"], d["kp"], d["vp"], d["kb"], d["vb"], d["ks"], d["vs"],
                              d["prefix_len"], out, d["h"], d["w"], conf, amax, tok, msk, w.tau,
                              commit_iter=citer, n_iters=nit)
    ws = dblock.alloc_workspace(dblock.decode_block_workspace_size(args), dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dblock.dblk_decode_block(args, ws, stream=torch.cuda.current_stream(), device=dev)
    for rep in range(3):
        tok.copy_(d["tokens"])
        msk.copy_(d["mask"])
        conf.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), eager["tokens"]), rep
        assert np.array_equal(citer.cpu().numpy(), eager["commit_iter"]), rep
        assert np.array_equal(nit.cpu().numpy(), eager["n_iters"]), rep
        # conf / argmax are promised on the positions masked at the start only
        m0 = inp["mask"].astype(bool)
        assert np.array_equal(conf.cpu().numpy()[m0], eager["conf"][m0]), rep
        _ = (d["h"].float() * 2).sum().item()              # unrelated eager work between replays


# ------------------------------------------------------------------ dual cache

@pytest.mark.parametrize("D,L,P_cap", [(64, 16, 128), (128, 64, 320), (128, 128, 4864)])
def test_cache_append_matches_oracle(D, L, P_cap):
    dev = require_gpu()
    B, H = 5, 3
    note(f"cache_append B={B} H={H} D={D} L={L} P_cap={P_cap}")
    rng = np.random.default_rng(D + L + P_cap)
    kp = rng.integers(0, 1 << 16, (B, H, P_cap, D), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, (B, H, P_cap, D), dtype=np.uint16)
    kb = rng.integers(0, 1 << 16, (B, H, L, D), dtype=np.uint16)
    vb = rng.integers(0, 1 << 16, (B, H, L, D), dtype=np.uint16)
    plen = np.array([0, P_cap // 3, P_cap - L, P_cap - L + 1, -4], dtype=np.int32)
    g = {k: bf16(v, dev) for k, v in (("kp", kp), ("vp", vp), ("kb", kb), ("vb", vb))}
    gl = torch.from_numpy(plen).to(dev)
    app = torch.empty(B, dtype=torch.int32, device=dev)
    dblock.dblk_cache_append(g["kp"], g["vp"], g["kb"], g["vb"], gl, app)
    torch.cuda.synchronize()
    rk, rv, rl, ra = cache_append(kp, vp, kb, vb, plen)
    as_bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(as_bits(g["kp"]), rk)
    assert np.array_equal(as_bits(g["vp"]), rv)
    assert np.array_equal(gl.cpu().numpy(), rl)
    assert np.array_equal(app.cpu().numpy(), ra)


def test_next_block_over_advanced_cache():
    """After the cache advance the next block's keys are the same rows as
    before, split differently: prefix' = prefix ++ block, block' = the first L
    suffix rows, suffix' = the rest of the suffix read in place (base pointer
    moved by L rows, row stride unchanged).  Attention through both layouts
    matches the oracle over the unsplit key set."""
    dev = require_gpu()
    w = custom_workload("adv", 35, B=3, H=4, D=128, L=32, P_cap=192, S=96, V=512)
    note("cache advance + suffix in place")
    inp = make_inputs(w)
    inp["prefix_len"] = np.array([40, 100, 160], dtype=np.int32)   # 160 + 32 = P_cap
    d = upload(inp, dev)
    B, H, L, D, S = w.B, w.H, w.L, w.D, w.S
    pl = d["prefix_len"].clone()
    kp, vp = d["kp"].clone(), d["vp"].clone()
    dblock.dblk_cache_append(kp, vp, d["kb"], d["vb"], pl)
    kb2 = d["ks"][:, :, :L].contiguous()
    vb2 = d["vs"][:, :, :L].contiguous()
    out = torch.empty_like(d["q"])
    ws = dblock.alloc_workspace(dblock.attend_workspace_size(B, H, L, D, w.P_cap, S - L), dev)
    lib = dblock.load_library()
    off = L * D * 2                                    # bytes: L rows of the suffix
    st = lib.dblk_attend(d["q"].data_ptr(), kp.data_ptr(), vp.data_ptr(), kb2.data_ptr(),
                         vb2.data_ptr(), d["ks"].data_ptr() + off, d["vs"].data_ptr() + off,
                         pl.data_ptr(), B, H, L, D, w.P_cap, S - L, S, 0.0, out.data_ptr(),
                         ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert pl.cpu().numpy().tolist() == [72, 132, 192]
    o = bf16_to_np(out)
    f = {k: bf16_bits_to_f64(inp[k]) for k in ("q", "kp", "vp", "kb", "vb", "ks", "vs")}
    ref = attend(f["q"], f["kp"], f["vp"], f["kb"], f["vb"], f["ks"], f["vs"], inp["prefix_len"])
    assert attention_row_rel_err(o, ref) <= 1e-2


@pytest.mark.parametrize("S", [0, 16, 128, 447])
def test_attend_suffix_window(S):
    """Suffix pruned to its first S rows of a 448-row buffer (read with the buffer's stride)."""
    dev = require_gpu()
    w = custom_workload("win", 36, B=1, H=16, D=128, L=64, P_cap=768, S=448, V=512)
    note(f"attend suffix window S={S} of {w.S}")
    inp = make_inputs(w)
    d = upload(inp, dev)
    out = torch.empty_like(d["q"])
    dblock.dblk_attend(d["q"], d["kp"], d["vp"], d["kb"], d["vb"], d["ks"], d["vs"],
                       d["prefix_len"], out, S=S)
    torch.cuda.synchronize()
    f = {k: bf16_bits_to_f64(inp[k]) for k in ("q", "kp", "vp", "kb", "vb", "ks", "vs")}
    ref = attend(f["q"], f["kp"], f["vp"], f["kb"], f["vb"], f["ks"][:, :, :S], f["vs"][:, :, :S],
                 inp["prefix_len"])
    assert attention_row_rel_err(bf16_to_np(out), ref) <= 1e-2
