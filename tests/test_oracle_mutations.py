"""The oracle's pins catch plausible mistakes in it.

Each case plants one mistake in a copy of the oracle's source (a dropped term,
a wrong index, axis or operand, a flipped comparison) and runs a compact set
of independent checks against the copy: scalar-Python brute force of the
attention, of the vocabulary softmax and of the decoder step over every mask
of a short block, scalar Python of a whole iteration over three ragged
sequences (explicit scale, a row subset), and exact bf16 decodes.  The unmodified oracle passes every
check; every planted mistake must fail at least one.  Nothing here runs on a
GPU and nothing is written to disk.
"""
import itertools
import math
import os
import types

import numpy as np
import pytest

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "dblock_oracle.py")


def _module(src: str) -> types.ModuleType:
    m = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), m.__dict__)
    return m


# ---- independent references (plain Python loops) ----

def _attention_case():
    rng = np.random.default_rng(7)
    B, H, L, D, P_cap, S = 2, 2, 3, 4, 5, 2
    f = lambda *s: rng.standard_normal(s)
    return dict(q=f(B, L, H, D), kp=f(B, H, P_cap, D), vp=f(B, H, P_cap, D), kb=f(B, H, L, D),
                vb=f(B, H, L, D), ks=f(B, H, S, D), vs=f(B, H, S, D),
                prefix_len=np.array([5, 2]))


def _attention_brute(c):
    q = c["q"]
    B, L, H, D = q.shape
    out = np.zeros((B, L, H, D))
    for b in range(B):
        P_b = int(c["prefix_len"][b])
        for h in range(H):
            keys = [c["kp"][b, h, t] for t in range(P_b)] + list(c["kb"][b, h]) + list(c["ks"][b, h])
            vals = [c["vp"][b, h, t] for t in range(P_b)] + list(c["vb"][b, h]) + list(c["vs"][b, h])
            for l in range(L):
                s = [sum(q[b, l, h, i] * k[i] for i in range(D)) / math.sqrt(D) for k in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for i in range(D):
                    out[b, l, h, i] = sum(e[j] * vals[j][i] for j in range(len(keys))) / z
    return out


def _vocab_case():
    rng = np.random.default_rng(11)
    M, d, V = 4, 3, 7
    h = rng.standard_normal((M, d))
    w = rng.standard_normal((V, d))
    w[5] = w[2]                        # row 0 of h ties tokens 2 and 5 exactly
    h[0] = w[2] * 3.0
    return h, w


def _vocab_brute(h, w):
    conf, amax, gap = [], [], []
    for r in range(h.shape[0]):
        logits = [sum(h[r, i] * w[t, i] for i in range(h.shape[1])) for t in range(w.shape[0])]
        m = max(logits)
        a = min(t for t, x in enumerate(logits) if x == m)
        z = sum(math.exp(x - m) for x in logits)
        conf.append(max(math.exp(x - m) / z for x in logits))
        amax.append(a)
        gap.append(m - max(x for t, x in enumerate(logits) if t != a))
    return np.array(conf), np.array(amax), np.array(gap)


def _commit_brute(conf_row, amax_row, tok_row, mask_row, tau):
    masked = [i for i in range(len(conf_row)) if mask_row[i]]
    C = [i for i in masked if conf_row[i] >= tau]
    if not C and masked:
        top = max(conf_row[i] for i in masked)
        C = [min(i for i in masked if conf_row[i] == top)]
    tok, msk = list(tok_row), list(mask_row)
    for i in C:
        tok[i], msk[i] = amax_row[i], 0
    return tok, msk, len(C)


# ---- the checks, each against a given copy of the oracle ----

def check_attention(m):
    c = _attention_case()
    o = m.attend(c["q"], c["kp"], c["vp"], c["kb"], c["vb"], c["ks"], c["vs"], c["prefix_len"])
    return np.abs(o - _attention_brute(c)).max() < 1e-12


def check_vocab(m):
    h, w = _vocab_case()
    conf, amax, gap = m.lmhead_confidence(h, w)
    rc, ra, rg = _vocab_brute(h, w)
    return (np.abs(conf - rc).max() < 1e-12 and (amax == ra).all()
            and np.abs(gap - rg).max() < 1e-12)


def check_commit(m):
    L = 5
    conf = np.array([[0.3, 0.9, 0.9, 0.2, 0.95]], dtype=np.float32)   # exact tie at and above tau
    amax = np.array([[11, 12, 13, 14, 15]])
    tok0 = np.array([[1, 2, 3, 4, 5]])
    for tau in (np.float32(0.9), np.float32(0.99), np.float32(0.0)):
        for bits in itertools.product((0, 1), repeat=L):
            mask = np.array([bits], dtype=np.uint8)
            tok, msk, n, _ = m.threshold_commit(conf, amax, tok0, mask, tau)
            rt, rm, rn = _commit_brute(conf[0], amax[0], tok0[0], mask[0], tau)
            if list(tok[0]) != rt or list(msk[0]) != rm or int(n[0]) != rn:
                return False
    return True


def check_bf16(m):
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x3EAB], dtype=np.uint16)
    want = np.array([1.0, -2.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, 0.333984375])
    return np.array_equal(m.bf16_bits_to_f64(bits), want)


def check_iteration(m):
    from tests.test_oracle_iteration import _brute_iteration, _tiny
    w, inp = _tiny()
    got = m.iteration(inp, w.tau, scale=0.37)
    ref = _brute_iteration(inp, w.tau, 0.37)
    if not (np.abs(got["o"] - ref["o"]).max() < 1e-12 and np.abs(got["conf"] - ref["conf"]).max() < 1e-12
            and got["argmax"].tolist() == ref["argmax"].tolist()
            and got["tokens"].tolist() == ref["tokens"].tolist()
            and got["mask"].tolist() == ref["mask"].tolist() and got["n"].tolist() == ref["n"].tolist()):
        return False
    rows = np.array([9, 0, 5, 11, 2])
    sub = m.iteration(inp, w.tau, rows=rows, with_attention=False)
    rs = _brute_iteration(inp, w.tau, 1.0, rows=rows)
    return np.abs(sub["conf"] - rs["conf"]).max() < 1e-12 and sub["argmax"].tolist() == rs["argmax"].tolist()


CHECKS = [check_attention, check_vocab, check_commit, check_bf16, check_iteration]


def _fails(m):
    failed = []
    for chk in CHECKS:
        try:
            ok = chk(m)
        except Exception:          # a crash is a caught mistake too
            ok = False
        if not ok:
            failed.append(chk.__name__)
    return failed


MUTATIONS = {
    "score scale 1/D": ("scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
    "softmax normalised over queries": ("p = e / e.sum(axis=1, keepdims=True)",
                                        "p = e / e.sum(axis=0, keepdims=True)"),
    "keys used as values": ("out[b, :, h, :] = p @ V", "out[b, :, h, :] = p @ K"),
    "ragged prefix not cut": ("K = np.concatenate([kp[b, h, :P_b]", "K = np.concatenate([kp[b, h]"),
    "suffix dropped": ("V = np.concatenate([vp[b, h, :P_b], vb[b, h], vs[b, h]], axis=0)",
                       "V = np.concatenate([vp[b, h, :P_b], vb[b, h]], axis=0)"),
    "vocabulary order reversed": ("        return h @ w.T\n", "        return (h @ w.T)[:, ::-1]\n"),
    "confidence is the sum, not its inverse": ("conf = 1.0 / S", "conf = S"),
    "max not subtracted in the exponent": ("S = np.exp(l - m[:, None]).sum(axis=1)",
                                           "S = np.exp(l).sum(axis=1)"),
    "argmax tie to the highest index": ("a = l.argmax(axis=1)",
                                        "a = l.shape[1] - 1 - l[:, ::-1].argmax(axis=1)"),
    "top-2 gap against the smallest logit": ("gap = m - rest.max(axis=1)",
                                             "gap = m - rest[np.isfinite(rest)].reshape(l.shape[0], -1).min(axis=1)"),
    "threshold exclusive": ("if conf[b, i] >= tau]", "if conf[b, i] > tau]"),
    "fallback takes the least confident": ("if conf[b, i] > conf[b, best]:", "if conf[b, i] < conf[b, best]:"),
    "fallback tie to the highest position": ("if conf[b, i] > conf[b, best]:", "if conf[b, i] >= conf[b, best]:"),
    "committed token is the position": ("tok[b, i] = argmax[b, i]", "tok[b, i] = i"),
    "committed positions stay masked": ("msk[b, i] = False", "msk[b, i] = msk[b, i]"),
    "fallback without a masked position": ("if not C and masked:", "if not C:"),
    "bf16 decoded with a 15-bit shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "iteration drops the score scale": ('inp["prefix_len"], scale)', 'inp["prefix_len"])'),
    "iteration ignores the row subset": ('lmhead_confidence(h, inp["w"], rows)',
                                         'lmhead_confidence(h, inp["w"])'),
    "iteration reshapes confidences sequence-minor": ("c32 = conf.astype(np.float32).reshape(B, L)",
                                                      "c32 = conf.astype(np.float32).reshape(L, B).T"),
    "iteration reshapes argmax sequence-minor": ("amax.reshape(B, L), inp[\"tokens\"]",
                                                 "amax.reshape(L, B).T, inp[\"tokens\"]"),
}


def test_unmodified_oracle_passes_every_check():
    with open(ORACLE_SRC) as f:
        assert _fails(_module(f.read())) == []


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name):
    with open(ORACLE_SRC) as f:
        src = f.read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    failed = _fails(_module(src.replace(old, new)))
    assert failed, f"no check catches: {name}"
