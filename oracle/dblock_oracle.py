"""fp64 CPU oracle of one denoising iteration of block-wise diffusion-LLM decoding.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Plain numpy in
float64, written from the definitions; no blocking, no online softmax, no
vocabulary splitting.  Every bf16 input is decoded exactly into float64.

What one iteration computes, and where the pages state it:

* dual KV cache -- the decoder is built with the dual KV-cache factory
  ("dInfer" GitHub README, usage section; the Fast-dLLM entry "Enabling KV
  Cache and Parallel Decoding" in the "Builds on" list of the dInfer index
  page): cached prefix and suffix keys/values are reused and only the active
  block is fresh.
* non-causal attention -- diffusion LLMs attend bidirectionally (topic page
  "Diffusion Language Model Inference", card view: the variable-size
  self-contained blocks abstract and the Streaming-dLLM abstract).
* confidence and argmax over the vocabulary, then the threshold parallel
  decoder -- a threshold-based parallel decoder with threshold 0.9 (README,
  usage section) and confidence-driven parallel decoding (DepCap abstract on
  the card-view topic page).

The pages do not write out the formulas; the readings taken here are:
score scale 1/sqrt(D); every block query sees every key of its row
(prefix[0:P_b] + block + suffix), no mask beyond the ragged prefix; softmax
over the full vocabulary at temperature 1 with no suppressed ids; confidence
is the largest softmax probability; argmax ties go to the lowest vocabulary
index; "meets the threshold" is conf >= tau; when no masked position meets it,
the single most confident masked position is committed (lowest position on an
exact tie); a row with nothing masked commits nothing.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns (uint16)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ attention

def dual_cache_kv(kp, vp, kb, vb, ks, vs, b: int, h: int, P_b: int) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values row (b, h) attends over: prefix[0:P_b], block, suffix.

    The dual cache of the README's usage section holds the prefix and the
    suffix; the block's own keys sit between them.
    """
    K = np.concatenate([kp[b, h, :P_b], kb[b, h], ks[b, h]], axis=0)
    V = np.concatenate([vp[b, h, :P_b], vb[b, h], vs[b, h]], axis=0)
    return K, V


def attend(q, kp, vp, kb, vb, ks, vs, prefix_len, scale: Optional[float] = None) -> np.ndarray:
    """Non-causal attention of the block's queries over the dual cache.

    q: [B][L][H][D]; kp/vp: [B][H][P_cap][D]; kb/vb: [B][H][L][D];
    ks/vs: [B][H][S][D]; prefix_len: [B].  All float64 (decoded bf16).
    Returns O [B][L][H][D] float64 with
    O = softmax(q K^T * scale) V per (b, h), no causal or other mask.
    """
    B, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, L, H, D), dtype=np.float64)
    for b in range(B):
        P_b = int(prefix_len[b])
        for h in range(H):
            K, V = dual_cache_kv(kp, vp, kb, vb, ks, vs, b, h, P_b)
            s = (q[b, :, h, :] @ K.T) * scale          # [L][T_b]
            # softmax; subtracting the row maximum leaves the value unchanged
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ V
    return out


# ------------------------------------------------------------------ LM head

def lm_logits(h: np.ndarray, w: np.ndarray, vchunk: int = 8192) -> np.ndarray:
    """Logits of the block's hidden states: l = h W^T (row t of W = token t).

    ``w`` is float64, or uint16 bf16 bit patterns; bit patterns are decoded
    exactly, ``vchunk`` vocabulary rows at a time into reused buffers (only to
    bound memory traffic; every logit is the same dot product).
    """
    if w.dtype != np.uint16:
        return h @ w.T
    V, d = w.shape
    out = np.empty((h.shape[0], V), dtype=np.float64)
    u32 = np.empty((min(vchunk, V), d), dtype=np.uint32)
    f64 = np.empty((min(vchunk, V), d), dtype=np.float64)
    for c0 in range(0, V, vchunk):
        c1 = min(V, c0 + vchunk)
        n = c1 - c0
        np.left_shift(w[c0:c1], 16, out=u32[:n], dtype=np.uint32)
        np.copyto(f64[:n], u32[:n].view(np.float32))
        out[:, c0:c1] = h @ f64[:n].T
    return out


def confidence_from_logits(logits: np.ndarray):
    """Per row: confidence (largest softmax probability), argmax, top-2 gap.

    conf = max_j exp(l_j) / sum_j exp(l_j) = 1 / sum_j exp(l_j - max l);
    argmax is the lowest index attaining max l; gap = max l minus the largest
    logit at any other index (0 on a tie).
    """
    l = np.atleast_2d(logits)
    m = l.max(axis=1)
    a = l.argmax(axis=1)                      # first occurrence = lowest index
    S = np.exp(l - m[:, None]).sum(axis=1)
    conf = 1.0 / S
    rest = l.copy()
    rest[np.arange(l.shape[0]), a] = -np.inf
    gap = m - rest.max(axis=1)
    return conf, a.astype(np.int64), gap


def lmhead_confidence(h: np.ndarray, w: np.ndarray, rows: Optional[np.ndarray] = None,
                      chunk: int = 64):
    """conf, argmax and top-2 gap for the rows of ``h`` (all rows by default).

    ``w`` is float64 or bf16 bit patterns (see ``lm_logits``).

    Rows are taken ``chunk`` at a time only to bound memory; each row's full
    logit vector exists at once, so this is the plain definition.
    """
    idx = np.arange(h.shape[0]) if rows is None else np.asarray(rows)
    conf = np.empty(len(idx)); amax = np.empty(len(idx), dtype=np.int64); gap = np.empty(len(idx))
    for s in range(0, len(idx), chunk):
        sel = idx[s:s + chunk]
        c, a, g = confidence_from_logits(lm_logits(h[sel], w))
        conf[s:s + chunk] = c; amax[s:s + chunk] = a; gap[s:s + chunk] = g
    return conf, amax, gap


# ------------------------------------------------------------------ commit

def threshold_commit(conf, argmax, tokens, mask, tau):
    """Threshold parallel decoding of one iteration, per sequence b.

    conf, argmax: [B][L]; tokens int [B][L]; mask bool/uint8 [B][L] (1 =
    still masked); tau: threshold, compared in the dtype of ``conf``.
    C = {i masked : conf_i >= tau}; if C is empty and some position is
    masked, C = {the masked position of highest confidence, lowest i on a
    tie}.  Committed positions take their argmax token and leave the mask.
    Returns (tokens', mask' uint8, n_committed int32 [B], fallback bool [B]).
    """
    conf = np.asarray(conf)
    tau = conf.dtype.type(tau)
    B, L = conf.shape
    tok = np.array(tokens, copy=True)
    msk = np.array(mask, dtype=bool, copy=True)
    n = np.zeros(B, dtype=np.int32)
    fb = np.zeros(B, dtype=bool)
    for b in range(B):
        masked = [i for i in range(L) if msk[b, i]]
        C = [i for i in masked if conf[b, i] >= tau]
        if not C and masked:
            best = masked[0]
            for i in masked[1:]:
                if conf[b, i] > conf[b, best]:
                    best = i
            C = [best]
            fb[b] = True
        for i in C:
            tok[b, i] = argmax[b, i]
            msk[b, i] = False
        n[b] = len(C)
    return tok, msk.astype(np.uint8), n, fb


# ------------------------------------------------------------------ iteration

def iteration(inp: Dict[str, np.ndarray], tau: float, scale: Optional[float] = None,
              rows: Optional[np.ndarray] = None, with_attention: bool = True):
    """One full iteration on generator inputs (bf16 bit patterns).

    Attention and the LM-head stage share no data (the transformer layers
    between them are outside this path).  The commit decision is taken in
    float32 (conf rounded to float32, tau as float32), the precision of the
    kernel that takes it.  ``rows`` restricts the LM head to a subset of the
    B*L rows (then tokens/mask are not computed).
    """
    res = {}
    if with_attention:
        f = {k: bf16_bits_to_f64(inp[k]) for k in ("q", "kp", "vp", "kb", "vb", "ks", "vs")}
        res["o"] = attend(f["q"], f["kp"], f["vp"], f["kb"], f["vb"], f["ks"], f["vs"],
                          inp["prefix_len"], scale)
    h = bf16_bits_to_f64(inp["h"])
    conf, amax, gap = lmhead_confidence(h, inp["w"], rows)
    res["conf"], res["argmax"], res["gap"] = conf, amax, gap
    if rows is None:
        B, L = inp["tokens"].shape
        c32 = conf.astype(np.float32).reshape(B, L)
        tok, msk, n, fb = threshold_commit(c32, amax.reshape(B, L), inp["tokens"],
                                           inp["mask"], np.float32(tau))
        res["tokens"], res["mask"], res["n"], res["fallback"] = tok, msk, n, fb
    return res
