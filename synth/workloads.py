"""Workload registry and seeded generator for the dual-cache decoding iteration.

Shapes follow the LLaDA / LLaDA-MoE usage described on the dInfer pages
(dInfer GitHub README, usage section: a threshold decoder at threshold 0.9
with the LLaDA-MoE mask and end-of-text ids, a dual KV cache, 1024 generated
tokens in blocks of 64, bf16 weights).  The pages run on public benchmarks (HumanEval and five more);
none of those items are used or reproduced here: every tensor is drawn from a
seeded distribution with the shape of the model it stands in for.

Input recipe (the same for every workload; only shapes and a few scalars vary):

* Q, K, V of every cache segment: N(0, 1), rounded to bf16 (RoPE is treated as
  already applied).
* LM-head W: N(0, 1/d), rounded to bf16, row t = token t.
* Block hidden states ("planted spike"): h_i = 0.5 z_i + a_i W[t_i] / ||W[t_i]||^2
  with z_i ~ N(0, I_d) independent per position, t_i uniform over the vocabulary,
  a_i ~ U[0, a_max], W[t_i] the bf16-rounded row; computed in fp64, rounded to
  fp32 and then to bf16.  The logit of t_i is then close to a_i.
* Mask: Bernoulli(p) per block position; a row with no masked position gets
  one uniformly chosen position flagged, so every row has work to commit.
* Tokens: unmasked positions hold uniform ids in [0, V); masked positions hold
  ``mask_id`` (156895 for the 157184-entry LLaDA-MoE vocabulary, V-1 otherwise).
* Ragged prefix (long-context workload): per-sequence prefix length
  P_b = U_int[lo, hi] + add, with the cache allocated at P_cap; rows of the
  prefix at t >= P_b hold random data that must never be read.

Every tensor has its own numpy ``SeedSequence(ROOT_SEED, spawn_key=...)`` stream
and large tensors are drawn in fixed 2**21-element chunks, each with its own
spawned stream, so values do not depend on thread count or on memory layout of
the draw.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np

ROOT_SEED = 20251009
CHUNK = 1 << 21

# Mask id of the LLaDA-MoE tokenizer as passed to the threshold decoder in the
# README's usage example; the pages give no mask id for LLaDA-8B.
LLADA_MOE_VOCAB = 157184
LLADA_MOE_MASK_ID = 156895

# tensor ids inside one workload's seed tree
_TID = {
    "q": 0, "kp": 1, "vp": 2, "kb": 3, "vb": 4, "ks": 5, "vs": 6,
    "w": 7, "z": 8, "t": 9, "a": 10, "mask": 11, "tokens": 12, "jitter": 13,
    "mask_fix": 14,
}


@dataclass(frozen=True)
class Workload:
    """One synthetic iteration: shapes, threshold and input distribution.

    B batch, H heads, D head dim (d = H*D), L block length, P_cap prefix
    capacity, S suffix length, V vocabulary, tau commit threshold, mask_p
    Bernoulli mask probability, a_max spike amplitude bound.
    """
    name: str
    B: int
    H: int
    D: int
    L: int
    P_cap: int
    S: int
    V: int
    tau: float
    mask_p: float
    a_max: float
    # (lo, hi, add): P_b = U_int[lo, hi] + add; None => P_b = P_cap for all b
    prefix_jitter: Optional[Tuple[int, int, int]] = None
    # seed-tree keys: tensors other than the mask share ``input_key``; the mask
    # and tokens use ``mask_key`` (so mask-fraction / threshold sweeps share
    # the rest of their inputs)
    input_key: Tuple[int, ...] = (99, 0)
    mask_key: Tuple[int, ...] = (99, 0)
    note: str = ""

    @property
    def d(self) -> int:
        return self.H * self.D

    @property
    def M(self) -> int:
        return self.B * self.L

    @property
    def T_cap(self) -> int:
        return self.P_cap + self.L + self.S

    @property
    def mask_id(self) -> int:
        return LLADA_MOE_MASK_ID if self.V == LLADA_MOE_VOCAB else self.V - 1

    def kv_bytes(self, prefix_len: Optional[np.ndarray] = None) -> int:
        """Bytes of K and V that one attention pass must read (bf16)."""
        if prefix_len is None:
            T = np.full(self.B, self.T_cap, dtype=np.int64)
        else:
            T = np.asarray(prefix_len, dtype=np.int64) + self.L + self.S
        return int(2 * self.H * self.D * 2 * T.sum())


def _c2(idx: int) -> Workload:
    # LLaDA-MoE-7B-A1B-shaped: prompt 256, gen 1024, block 64 at block index idx
    return Workload(
        name=f"c2-blk{idx}", B=1, H=16, D=128, L=64,
        P_cap=256 + 64 * idx, S=1024 - 64 * (idx + 1), V=157184,
        tau=0.9, mask_p=0.5, a_max=24.0,
        input_key=(2, idx), mask_key=(2, idx),
        note="LLaDA-MoE-7B-A1B-shaped, block index %d" % idx)


def _c1(pct: int) -> Workload:
    return Workload(
        name=f"c1-mask{pct}", B=1, H=32, D=128, L=64, P_cap=1024, S=512,
        V=126464, tau=0.9, mask_p=pct / 100.0, a_max=24.0,
        input_key=(1, 0), mask_key=(1, pct),
        note="LLaDA-8B-shaped, mask fraction %d%%" % pct)


def _c4(tau_pct: int) -> Workload:
    return Workload(
        name=f"c4-tau{tau_pct}", B=32, H=16, D=128, L=128, P_cap=1024, S=1536,
        V=157184, tau=tau_pct / 100.0, mask_p=0.3, a_max=24.0,
        input_key=(4, 0), mask_key=(4, 0),
        note="throughput batch 32, threshold %.2f" % (tau_pct / 100.0))


def _registry() -> Dict[str, Workload]:
    w = {}
    w["c0"] = Workload(
        name="c0", B=1, H=4, D=64, L=32, P_cap=128, S=64, V=4096,
        tau=0.9, mask_p=0.5, a_max=20.0, input_key=(0, 0), mask_key=(0, 0),
        note="tiny, CPU-seconds")
    for pct in (100, 50, 10):
        w[f"c1-mask{pct}"] = _c1(pct)
    for idx in (0, 8, 15):
        w[f"c2-blk{idx}"] = _c2(idx)
    w["c3"] = Workload(
        name="c3", B=8, H=32, D=128, L=64, P_cap=4864, S=256, V=126464,
        tau=0.9, mask_p=0.5, a_max=24.0, prefix_jitter=(3584, 4096, 768),
        input_key=(3, 0), mask_key=(3, 0),
        note="long context batch 8, ragged prefix")
    for tp in (70, 90, 95):
        w[f"c4-tau{tp}"] = _c4(tp)
    # secondary readings of the suffix length: gen - (index+1)*block
    w["c1-mask50-dS"] = replace(w["c1-mask50"], name="c1-mask50-dS", S=448,
                                note="LLaDA-8B-shaped, derived suffix 448")
    w["c3-dS"] = replace(w["c3"], name="c3-dS", S=192, note="c3 with derived suffix 192")
    w["c4-tau90-dS"] = replace(w["c4-tau90"], name="c4-tau90-dS", S=1408,
                               note="c4 with derived suffix 1408")
    return w


WORKLOADS: Dict[str, Workload] = _registry()
PRIMARY = ["c0", "c1-mask100", "c1-mask50", "c1-mask10", "c2-blk0", "c2-blk8",
           "c2-blk15", "c3", "c4-tau70", "c4-tau90", "c4-tau95"]


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom_workload(name: str, key: int, **kw) -> Workload:
    """A small ad-hoc workload for tests (own seed tree ``(100 + key, 0)``)."""
    base = dict(B=1, H=2, D=64, L=16, P_cap=32, S=16, V=512, tau=0.9,
                mask_p=0.5, a_max=20.0)
    base.update(kw)
    return Workload(name=name, input_key=(100 + key, 0), mask_key=(100 + key, 0), **base)


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits.

    Inputs must be finite (the generator never makes NaN or Inf).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- streams

def _rng(key: Tuple[int, ...], tensor: str, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(key) + (_TID[tensor], sub)))


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _normal_bf16(key, tensor: str, shape, scale: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, scale^2) with the given shape, drawn chunk by chunk."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK
    sc = np.float32(scale)

    def fill(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        x = _rng(key, tensor, 1 + c).standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= sc
        out[lo:hi] = f32_to_bf16_bits(x)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# ---------------------------------------------------------------- generator

def make_inputs(w: Workload, parts=("attn", "lmhead", "commit")) -> Dict[str, np.ndarray]:
    """Draw every input of one iteration of workload ``w``.

    Returns numpy arrays; bf16 tensors are uint16 bit patterns:

    * ``q`` [B][L][H][D]; ``kp``/``vp`` [B][H][P_cap][D]; ``kb``/``vb``
      [B][H][L][D]; ``ks``/``vs`` [B][H][S][D]; ``prefix_len`` int32 [B]
    * ``w`` [V][d]; ``h`` [B*L][d]; ``t`` int64 [B*L]; ``a`` float64 [B*L]
    * ``tokens`` int32 [B][L]; ``mask`` uint8 [B][L] (1 = still masked)
    """
    out: Dict[str, np.ndarray] = {}
    B, H, D, L, V, d = w.B, w.H, w.D, w.L, w.V, w.d
    ik, mk = w.input_key, w.mask_key
    if "attn" in parts:
        out["q"] = _normal_bf16(ik, "q", (B, L, H, D))
        out["kp"] = _normal_bf16(ik, "kp", (B, H, w.P_cap, D))
        out["vp"] = _normal_bf16(ik, "vp", (B, H, w.P_cap, D))
        out["kb"] = _normal_bf16(ik, "kb", (B, H, L, D))
        out["vb"] = _normal_bf16(ik, "vb", (B, H, L, D))
        out["ks"] = _normal_bf16(ik, "ks", (B, H, w.S, D))
        out["vs"] = _normal_bf16(ik, "vs", (B, H, w.S, D))
        if w.prefix_jitter is None:
            pl = np.full(B, w.P_cap, dtype=np.int32)
        else:
            lo, hi, add = w.prefix_jitter
            pl = (_rng(ik, "jitter").integers(lo, hi + 1, size=B) + add).astype(np.int32)
            assert pl.max() <= w.P_cap
        out["prefix_len"] = pl
    if "lmhead" in parts:
        W = _normal_bf16(ik, "w", (V, d), scale=1.0 / np.sqrt(d))
        out["w"] = W
        M = B * L
        z = _rng(ik, "z").standard_normal((M, d))
        t = _rng(ik, "t").integers(0, V, size=M)
        a = _rng(ik, "a").uniform(0.0, w.a_max, size=M)
        rows = bf16_bits_to_f32(W[t]).astype(np.float64)
        nrm2 = np.einsum("ij,ij->i", rows, rows)
        hf = 0.5 * z + (a / nrm2)[:, None] * rows
        out["h"] = f32_to_bf16_bits(hf.astype(np.float32))
        out["t"] = t
        out["a"] = a
    if "commit" in parts:
        mask = _rng(mk, "mask").random((B, L)) < w.mask_p
        fix = _rng(mk, "mask_fix")
        for b in range(B):
            if not mask[b].any():
                mask[b, fix.integers(0, L)] = True
        tokens = _rng(mk, "tokens").integers(0, V, size=(B, L)).astype(np.int32)
        tokens[mask] = w.mask_id
        out["mask"] = mask.astype(np.uint8)
        out["tokens"] = tokens
    return out
