"""Whole iteration (attend -> LM head/confidence -> threshold commit) vs the
fp64 oracle on every workload at full size.

The GPU runs the full iteration exactly as the benchmark launches it.  The
oracle computes what it can in seconds: every row and every (b, h) when the
workload is small; otherwise every block row of a few sampled sequences (the
commit decision needs a whole sequence) and a sample of (b, h) attention rows,
always including the shortest and longest ragged prefix.

Bars: attention per-row relative error <= 1e-2; confidence within 1e-3
absolute; argmax identical where the oracle's top-2 gap >= 1e-3; committed
tokens and updated mask identical outside the excluded set E (oracle
confidence within 1e-3 of the threshold, top-2 gap below 1e-3, or a fallback
decided by a near-tie); |E| is printed.
"""
import numpy as np
import pytest

from oracle import (attend, attention_row_rel_err, bf16_bits_to_f64, compare_commit,
                    exclusion_set, lmhead_confidence, threshold_commit)
from synth import WORKLOADS, make_inputs
from synth.workloads import PRIMARY
from tests.gpu_util import note, require_gpu, run_iteration, upload

pytestmark = pytest.mark.gpu

VARIANTS = PRIMARY + ["c1-mask50-dS", "c3-dS", "c4-tau90-dS"]
_cache = {}


def _inputs(w):
    key = (w.input_key, w.mask_key, w.S, w.P_cap, w.B, w.L, w.V)
    if key not in _cache:
        _cache.clear()
        _cache[key] = make_inputs(w)
    return _cache[key]


def _sample_seqs(w, inp):
    if w.M <= 128:
        return list(range(w.B))
    pl = inp["prefix_len"]
    return sorted({0, w.B - 1, int(np.argmin(pl)), int(np.argmax(pl))})[:3]


def _sample_bh(w, inp, seqs):
    if w.B * w.H <= 64:
        return [(b, h) for b in range(w.B) for h in range(w.H)]
    rng = np.random.default_rng(w.B * 131 + w.H)
    out = [(b, h) for b in seqs for h in (0, w.H - 1)]
    out += [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(8)]
    return sorted(set(out))


@pytest.mark.parametrize("name", VARIANTS)
def test_iteration(name):
    dev = require_gpu()
    w = WORKLOADS[name]
    note(f"iteration {name}: B={w.B} H={w.H} D={w.D} L={w.L} P_cap={w.P_cap} S={w.S} V={w.V} tau={w.tau}")
    inp = _inputs(w)
    g = run_iteration(upload(inp, dev), w.tau)

    # -------- attention on sampled (b, h)
    seqs = _sample_seqs(w, inp)
    errs = []
    for b, h in _sample_bh(w, inp, seqs):
        sl = lambda k: bf16_bits_to_f64(inp[k][b:b + 1, h:h + 1])
        q = bf16_bits_to_f64(inp["q"][b:b + 1, :, h:h + 1])
        ref = attend(q, sl("kp"), sl("vp"), sl("kb"), sl("vb"), sl("ks"), sl("vs"),
                     inp["prefix_len"][b:b + 1])
        errs.append(attention_row_rel_err(g["o"][b:b + 1, :, h:h + 1], ref))
    aerr = max(errs)

    # -------- LM head on every row of the sampled sequences
    rows = np.concatenate([np.arange(b * w.L, (b + 1) * w.L) for b in seqs])
    rc, ra, rg = lmhead_confidence(bf16_bits_to_f64(inp["h"]), inp["w"], rows=rows)
    cerr = float(np.abs(g["conf"][rows] - rc).max())
    ok = rg >= 1e-3
    amis = int((g["argmax"][rows][ok] != ra[ok]).sum())

    # -------- commit on the sampled sequences
    nb = len(seqs)
    conf_ref = rc.reshape(nb, w.L)
    tok_in = inp["tokens"][seqs]
    msk_in = inp["mask"][seqs]
    rt, rm, rn, rfb = threshold_commit(conf_ref.astype(np.float32), ra.reshape(nb, w.L), tok_in,
                                       msk_in, np.float32(w.tau))
    E = exclusion_set(conf_ref, rg.reshape(nb, w.L), msk_in, w.tau)
    bad = compare_commit(g["tokens"][seqs], g["mask"][seqs], rt, rm, E)
    committed = int((msk_in.astype(bool) & ~g["mask"][seqs].astype(bool)).sum())
    note(f"  attn err={aerr:.2e} over {len(errs)} (b,h); conf err={cerr:.2e}; argmax mismatches="
         f"{amis} (excluded {int((~ok).sum())}); commit mismatches={bad}; |E|={int(E.sum())} of "
         f"{E.size}; committed={committed} (oracle {int(rn.sum())}); fallback rows={int(rfb.sum())}")
    assert aerr <= 1e-2
    assert cerr <= 1e-3
    assert amis == 0
    assert bad == 0
    # invariants on every sequence of the GPU result
    m_in = inp["mask"].astype(bool)
    m_out = g["mask"].astype(bool)
    assert not (m_out & ~m_in).any()                                   # only masked positions commit
    assert ((m_in & ~m_out).sum(axis=1) >= 1).all()                    # at least one per sequence
    np.testing.assert_array_equal(g["tokens"][m_out | ~m_in], inp["tokens"][m_out | ~m_in])
    assert (g["n"] == (m_in & ~m_out).sum(axis=1)).all()
