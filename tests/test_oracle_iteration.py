"""Pins for the oracle's whole iteration (CPU only).

``oracle.iteration`` glues the pinned pieces together: it decodes the bf16
generator inputs, runs the attention over every (b, h), the LM head over the
B*L block rows and the decoder step per sequence.  What can go wrong there is
the glue: a batch reshape, a scale that is not passed through, a row subset
taken in the wrong order, the commit taken on another sequence's rows.  Two
independent references catch those:

* scalar Python (``math.exp`` loops, bf16 decoded with ``struct``) of the
  whole iteration on a tiny batch of three sequences with ragged prefixes,
  an explicit score scale and a row subset in scrambled order;
* per-sequence compositions of the pinned ``attend``, ``lmhead_confidence``
  and ``threshold_commit`` at a size that spans several sequences of 32 rows.

The definitions followed are those of the oracle's header: dual-cache
attention (dInfer README, usage section, the 'dual' KV-cache factory),
softmax confidence over the vocabulary and the threshold decoder (README,
usage section, ThresholdParallelDecoder; DepCap abstract on the topic page).
"""
import math
import struct

import numpy as np
import pytest

from oracle import attend, bf16_bits_to_f64, iteration, lmhead_confidence, threshold_commit
from synth import custom_workload, make_inputs


def _bf16(bits) -> float:
    """Exact value of one bfloat16 bit pattern: it is the top half of a float32."""
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _tiny():
    w = custom_workload("it-tiny", 61, B=3, H=2, D=4, L=4, P_cap=6, S=2, V=24, tau=0.6,
                        mask_p=0.6, a_max=8.0, prefix_jitter=(0, 6, 0))
    inp = make_inputs(w)
    # the draw must exercise ragged prefixes, including an empty one
    inp["prefix_len"] = np.array([6, 0, 3], dtype=np.int32)
    return w, inp


def _brute_iteration(inp, tau, scale, rows=None):
    """The whole iteration in scalar Python, from the definitions."""
    q = inp["q"]
    B, L, H, D = q.shape
    P = inp["prefix_len"]
    o = np.zeros((B, L, H, D))
    for b in range(B):
        for h in range(H):
            keys = ([[_bf16(x) for x in inp["kp"][b, h, t]] for t in range(int(P[b]))]
                    + [[_bf16(x) for x in r] for r in inp["kb"][b, h]]
                    + [[_bf16(x) for x in r] for r in inp["ks"][b, h]])
            vals = ([[_bf16(x) for x in inp["vp"][b, h, t]] for t in range(int(P[b]))]
                    + [[_bf16(x) for x in r] for r in inp["vb"][b, h]]
                    + [[_bf16(x) for x in r] for r in inp["vs"][b, h]])
            for l in range(L):
                qv = [_bf16(x) for x in q[b, l, h]]
                s = [scale * sum(qv[i] * k[i] for i in range(D)) for k in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for i in range(D):
                    o[b, l, h, i] = sum(e[j] * vals[j][i] for j in range(len(keys))) / z
    hid, Wt = inp["h"], inp["w"]
    V, d = Wt.shape
    Wf = [[_bf16(x) for x in Wt[t]] for t in range(V)]
    idx = list(range(B * L)) if rows is None else [int(r) for r in rows]
    conf, amax, gap = [], [], []
    for r in idx:
        hv = [_bf16(x) for x in hid[r]]
        lg = [sum(hv[k] * Wf[t][k] for k in range(d)) for t in range(V)]
        m = max(lg)
        a = min(t for t in range(V) if lg[t] == m)
        conf.append(1.0 / sum(math.exp(x - m) for x in lg))
        amax.append(a)
        gap.append(m - max(lg[t] for t in range(V) if t != a))
    res = {"o": o, "conf": np.array(conf), "argmax": np.array(amax), "gap": np.array(gap)}
    if rows is None:
        tok = inp["tokens"].copy()
        msk = inp["mask"].copy()
        n = np.zeros(B, dtype=np.int32)
        t32 = float(np.float32(tau))
        for b in range(B):
            c32 = [float(np.float32(conf[b * L + i])) for i in range(L)]
            masked = [i for i in range(L) if msk[b, i]]
            C = [i for i in masked if c32[i] >= t32]
            if not C and masked:
                top = max(c32[i] for i in masked)
                C = [min(i for i in masked if c32[i] == top)]
            for i in C:
                tok[b, i] = amax[b * L + i]
                msk[b, i] = 0
            n[b] = len(C)
        res.update(tokens=tok, mask=msk, n=n)
    return res


@pytest.mark.parametrize("scale", [None, 0.37])
def test_iteration_matches_scalar_brute_force(scale):
    w, inp = _tiny()
    got = iteration(inp, w.tau, scale=scale)
    ref = _brute_iteration(inp, w.tau, 1.0 / math.sqrt(w.D) if scale is None else scale)
    np.testing.assert_allclose(got["o"], ref["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["conf"], ref["conf"], rtol=1e-12)
    assert got["argmax"].tolist() == ref["argmax"].tolist()
    np.testing.assert_allclose(got["gap"], ref["gap"], rtol=1e-10, atol=1e-12)
    assert got["tokens"].tolist() == ref["tokens"].tolist()
    assert got["mask"].tolist() == ref["mask"].tolist()
    assert got["n"].tolist() == ref["n"].tolist()
    # the draw has a commit in every sequence and leaves something masked
    assert (got["n"] >= 1).all() and got["mask"].any()


def test_scale_changes_the_output():
    # guards the comparison above against a scale that is silently ignored
    w, inp = _tiny()
    a = iteration(inp, w.tau, scale=0.37)["o"]
    b = iteration(inp, w.tau)["o"]
    assert np.abs(a - b).max() > 1e-3


def test_row_subset_in_given_order():
    w, inp = _tiny()
    rows = np.array([9, 0, 5, 11, 2])
    got = iteration(inp, w.tau, rows=rows, with_attention=False)
    ref = _brute_iteration(inp, w.tau, 1.0, rows=rows)
    np.testing.assert_allclose(got["conf"], ref["conf"], rtol=1e-12)
    assert got["argmax"].tolist() == ref["argmax"].tolist()
    assert "tokens" not in got and "o" not in got


def test_iteration_is_the_per_sequence_composition():
    # four sequences of 32 rows, ragged prefixes, explicit scale: every
    # sequence's outputs equal the pinned pieces called on that sequence alone
    w = custom_workload("it-comp", 62, B=4, H=3, D=64, L=32, P_cap=80, S=24, V=3000,
                        tau=0.8, mask_p=0.5, prefix_jitter=(10, 80, 0))
    inp = make_inputs(w)
    assert len(set(inp["prefix_len"].tolist())) > 1
    scale = 0.11
    got = iteration(inp, w.tau, scale=scale)
    hf = bf16_bits_to_f64(inp["h"])
    for b in range(w.B):
        f = {k: bf16_bits_to_f64(inp[k][b:b + 1]) for k in ("q", "kp", "vp", "kb", "vb", "ks", "vs")}
        o = attend(f["q"], f["kp"], f["vp"], f["kb"], f["vb"], f["ks"], f["vs"],
                   inp["prefix_len"][b:b + 1], scale)
        np.testing.assert_allclose(got["o"][b:b + 1], o, rtol=1e-13, atol=1e-15)
        c, a, g = lmhead_confidence(hf[b * w.L:(b + 1) * w.L], inp["w"])
        np.testing.assert_allclose(got["conf"][b * w.L:(b + 1) * w.L], c, rtol=1e-13)
        assert got["argmax"][b * w.L:(b + 1) * w.L].tolist() == a.tolist()
        tok, msk, n, fb = threshold_commit(c.astype(np.float32)[None], a[None],
                                           inp["tokens"][b:b + 1], inp["mask"][b:b + 1],
                                           np.float32(w.tau))
        assert got["tokens"][b].tolist() == tok[0].tolist()
        assert got["mask"][b].tolist() == msk[0].tolist()
        assert int(got["n"][b]) == int(n[0]) and bool(got["fallback"][b]) == bool(fb[0])
