"""fp64 CPU oracle of what surrounds one iteration: end-of-text handling, the
loop over a block's iterations, and the dual-cache advance at block end.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Plain numpy and
Python loops, written from the definitions below.

Where the pages state it:

* the block loop -- the block-wise diffusion generator produces 1024 tokens
  in blocks of 64, block after block ("dInfer" GitHub README, usage
  section); within a block, denoising iterations repeat
  until no masked position is left, each one committing at least one position
  (the threshold decoder's fallback), and dInfer unrolls these iterations on
  the device to avoid stream bubbles (README overview: loop unrolling and CUDA
  Graphs).
* end of text -- the decoder is given an ``eos_id`` (README usage section);
  what it does with it is not described.
* the dual cache -- the dual KV-cache factory (README usage section): prefix
  and suffix keys/values are cached around the active block.

Readings taken where the pages are silent:

* EOS: nothing but EOS follows an EOS.  After a decoder step, let e be the
  lowest unmasked position of the row holding eos_id; every still-masked
  position after e is committed as eos_id, and the row is "finished".
* Block loop: the layers that would produce new hidden states are outside
  the path, so every iteration sees the same confidences; the loop runs until
  the mask is empty or a given number of iterations has run.
* Cache advance: the completed block's keys/values are appended after each
  sequence's valid prefix rows; a sequence whose prefix would outgrow the
  buffer is left unchanged.  The suffix of the next block is the old one
  without its first L rows (no arithmetic, a view).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .dblock_oracle import threshold_commit


def threshold_commit_eos(conf, argmax, tokens, mask, tau, eos_id: int):
    """Decoder step, then the end-of-text rule, per sequence b.

    Returns (tokens', mask' uint8, n_committed int32 [B], fallback bool [B],
    finished uint8 [B]); n_committed counts threshold, fallback and EOS-fill
    commits together.
    """
    tok, msk, n, fb = threshold_commit(conf, argmax, tokens, mask, tau)
    msk = msk.astype(bool)
    B, L = tok.shape
    finished = np.zeros(B, dtype=np.uint8)
    for b in range(B):
        e = None
        for i in range(L):
            if not msk[b, i] and tok[b, i] == eos_id:
                e = i
                break
        if e is None:
            continue
        finished[b] = 1
        for i in range(e + 1, L):
            if msk[b, i]:
                tok[b, i] = eos_id
                msk[b, i] = False
                n[b] += 1
    return tok, msk.astype(np.uint8), n, fb, finished


def decode_block(conf, argmax, tokens, mask, tau, eos_id: Optional[int] = None,
                 max_iters: Optional[int] = None):
    """Iterations of one block on unchanging confidences.

    conf [B][L] (compared with tau in its own dtype), argmax [B][L], tokens,
    mask as for threshold_commit.  Runs max_iters steps (default L, which is
    always enough: every step commits at least one position of every row
    that has one).
    Returns (tokens', mask', commit_iter int32 [B][L] (-1: not committed),
    n_iters int32 [B] (1 + index of the row's last committing step),
    finished uint8 [B] (zeros without EOS handling)).
    """
    conf = np.asarray(conf)
    B, L = conf.shape
    iters = L if (max_iters is None or max_iters <= 0) else int(max_iters)
    tok = np.array(tokens, copy=True)
    msk = np.array(mask, dtype=bool, copy=True)
    commit_iter = np.full((B, L), -1, dtype=np.int32)
    n_iters = np.zeros(B, dtype=np.int32)
    finished = np.zeros(B, dtype=np.uint8)
    for t in range(iters):
        if eos_id is None:
            tok2, msk2, n, _ = threshold_commit(conf, argmax, tok, msk, tau)
        else:
            tok2, msk2, n, _, finished = threshold_commit_eos(conf, argmax, tok, msk, tau, eos_id)
        msk2 = msk2.astype(bool)
        commit_iter[msk & ~msk2] = t
        n_iters[n > 0] = t + 1
        tok, msk = tok2, msk2
    return tok, msk.astype(np.uint8), commit_iter, n_iters, finished


def cache_append(kp, vp, kb, vb, prefix_len):
    """Dual-cache advance at block end.

    kp, vp [B][H][P_cap][D]; kb, vb [B][H][L][D]; prefix_len [B].  With P_b =
    prefix_len[b] clipped to [0, P_cap]: if P_b + L <= P_cap, rows
    P_b .. P_b+L-1 of sequence b's prefix become the block's rows and its
    prefix length becomes P_b + L.  Returns new (kp, vp, prefix_len int32,
    appended int32 [B] = L or 0); the inputs are not modified.
    """
    kp = np.array(kp, copy=True)
    vp = np.array(vp, copy=True)
    B, H, P_cap, _ = kp.shape
    L = kb.shape[2]
    plen = np.array(prefix_len, dtype=np.int64).reshape(B)
    new_len = np.zeros(B, dtype=np.int32)
    appended = np.zeros(B, dtype=np.int32)
    for b in range(B):
        P_b = min(max(int(plen[b]), 0), P_cap)
        if P_b + L <= P_cap:
            kp[b, :, P_b:P_b + L] = kb[b]
            vp[b, :, P_b:P_b + L] = vb[b]
            new_len[b] = P_b + L
            appended[b] = L
        else:
            new_len[b] = P_b
    return kp, vp, new_len, appended
