"""Comparison rules between the HIP path and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (used by the tests, the smoke check and the bench's
CPU-baseline leg).

* Committed tokens and the updated mask must match bit for bit, except on the
  excluded set E: positions whose oracle confidence lies within ``band`` of the
  threshold, positions whose oracle top-2 logit gap is below ``band``, and,
  in a row where the oracle's at-least-one fallback fired, the two most
  confident masked positions if their oracle confidences differ by less than
  ``band`` (a near-tie decides which one is committed).
* Attention: per output row (b, l, h), max-abs error over max-abs reference,
  maximised over rows.
"""
from __future__ import annotations

import numpy as np


def exclusion_set(conf_ref, gap_ref, mask_in, tau, band: float = 1e-3):
    """Boolean [B][L]: positions excluded from the exact commit comparison."""
    conf_ref = np.asarray(conf_ref, dtype=np.float64)
    gap_ref = np.asarray(gap_ref, dtype=np.float64)
    m = np.asarray(mask_in, dtype=bool)
    E = (np.abs(conf_ref - float(tau)) < band) | (gap_ref < band)
    B, L = conf_ref.shape
    for b in range(B):
        idx = np.flatnonzero(m[b])
        if idx.size == 0:
            continue
        c = conf_ref[b, idx]
        if (c >= float(tau)).any():
            continue            # the oracle's threshold set is non-empty: no fallback
        order = np.argsort(-c, kind="stable")
        if idx.size >= 2 and c[order[0]] - c[order[1]] < band:
            E[b, idx[order[0]]] = True
            E[b, idx[order[1]]] = True
    return E


def compare_commit(tok_gpu, mask_gpu, tok_ref, mask_ref, E):
    """Number of mismatching non-excluded positions (tokens or mask)."""
    keep = ~np.asarray(E, dtype=bool)
    bad = (np.asarray(tok_gpu) != np.asarray(tok_ref)) | (
        np.asarray(mask_gpu).astype(bool) != np.asarray(mask_ref).astype(bool))
    return int((bad & keep).sum())


def attention_row_rel_err(o_gpu, o_ref) -> float:
    """max over (b,l,h) of ||o_gpu - o_ref||_inf / ||o_ref||_inf over D."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    num = np.abs(o_gpu - o_ref).max(axis=-1)
    den = np.abs(o_ref).max(axis=-1)
    return float((num / np.maximum(den, 1e-300)).max())


def block_schedule_violations(conf_ref, mask0, tau, commit_iter, n_iters, band: float = 1e-3):
    """Checks a block loop's schedule (no EOS handling) against the decoder's rules.

    The schedule is valid if it is what the decoder does on SOME confidences
    within ``band`` of the reference ones, kept fixed over the iterations:
    step 0 commits every masked position that surely meets the threshold and
    only positions that may meet it, or, when none surely does, one position
    that may be the most confident; every later step commits exactly one
    position that may be the most confident of those left and that surely
    did not meet the threshold; every masked position gets committed;
    n_iters = 1 + the last step's index.  Returns a list of violations.
    """
    c = np.asarray(conf_ref, dtype=np.float64)
    m = np.asarray(mask0, dtype=bool)
    g = np.asarray(commit_iter)
    n_it = np.asarray(n_iters)
    tau = float(tau)
    errs = []
    B, _ = c.shape
    for b in range(B):
        idx = np.flatnonzero(m[b])
        if (g[b, ~m[b]] != -1).any():
            errs.append(f"row {b}: an unmasked position was committed")
        if idx.size == 0:
            if n_it[b] != 0:
                errs.append(f"row {b}: nothing masked but n_iters = {n_it[b]}")
            continue
        gb, cb = g[b, idx], c[b, idx]
        if (gb < 0).any():
            errs.append(f"row {b}: {(gb < 0).sum()} masked positions never committed")
            continue
        sure = cb >= tau + band
        maybe = cb >= tau - band
        first = gb == 0
        threshold_step = first.any() and maybe[first].all() and first[sure].all()
        fallback_step = (not sure.any()) and first.sum() == 1 and cb[first][0] >= cb.max() - band
        if not (threshold_step or fallback_step):
            errs.append(f"row {b}: step 0 committed positions {idx[first].tolist()}")
        last = int(gb.max())
        for t in range(1, last + 1):
            sel = np.flatnonzero(gb == t)
            if sel.size != 1:
                errs.append(f"row {b}: step {t} committed {sel.size} positions")
                continue
            left = cb[gb >= t]
            if cb[sel[0]] < left.max() - band or sure[sel[0]]:
                errs.append(f"row {b}: step {t} committed position {idx[sel[0]]}")
        if n_it[b] != last + 1:
            errs.append(f"row {b}: n_iters {n_it[b]} != {last + 1}")
    return errs


def block_schedule_unambiguous(conf_ref, mask0, tau, band: float = 1e-3):
    """Bool [B]: rows whose schedule no confidence within ``band`` can change.

    A row is ambiguous if a masked confidence lies within ``band`` of the
    threshold, or if two masked positions that may be committed by the
    fallback (confidence below tau + band) lie within ``band`` of each other.
    """
    c = np.asarray(conf_ref, dtype=np.float64)
    m = np.asarray(mask0, dtype=bool)
    tau = float(tau)
    out = np.ones(c.shape[0], dtype=bool)
    for b in range(c.shape[0]):
        cb = c[b, m[b]]
        if (np.abs(cb - tau) < band).any():
            out[b] = False
            continue
        f = np.sort(cb[cb < tau + band])
        if f.size >= 2 and (np.diff(f) < band).any():
            out[b] = False
    return out
