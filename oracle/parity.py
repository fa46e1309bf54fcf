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
