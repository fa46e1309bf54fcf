"""dblk_attend_segments (strided segments, per-sequence lengths) vs the fp64 oracle.

The operation is dblk_attend's -- non-causal attention of the block over the
dual cache (dInfer README, usage section, the 'dual' KV-cache factory) -- with
every tensor given by element strides: q taken from a fused QKV projection
[B][L][3][H][D], caches stored head-interleaved [B][T][H][D], block keys and
values read straight out of the fused projection, output written into a
strided view, ragged prefix, block and suffix lengths per sequence.

The oracle sees the same values laid out densely, one sequence at a time
(the rows each sequence attends), so layout and length handling are checked
against the plain definition.  Bars: per-row relative error <= 1e-2;
dense views give results bit-identical to dblk_attend; a sequence with no
key at all is written as zeros (the call's stated convention); elements of
the output buffer outside the view are never written.
"""
import numpy as np
import pytest
import torch

from block_wise_decoding_amd import dblock
from oracle import attend, attention_row_rel_err, bf16_bits_to_f64
from synth import WORKLOADS, make_inputs
from synth.workloads import f32_to_bf16_bits
from tests.gpu_util import bf16, bf16_to_np, note, require_gpu, upload

pytestmark = pytest.mark.gpu


def _bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _oracle_rows(q, kp, vp, kb, vb, ks, vs, P, Lk, S):
    """Per-sequence oracle on dense float64 arrays: q [B][L][H][D],
    caches [B][H][T][D]; sequence b attends prefix[:P[b]] ++ block[:Lk[b]] ++ suffix[:S[b]]."""
    B = q.shape[0]
    out = np.zeros(q.shape)
    for b in range(B):
        if P[b] + Lk[b] + S[b] == 0:
            continue                       # no key: the call writes zeros
        out[b:b + 1] = attend(q[b:b + 1], kp[b:b + 1], vp[b:b + 1], kb[b:b + 1, :, :Lk[b]],
                              vb[b:b + 1, :, :Lk[b]], ks[b:b + 1, :, :S[b]], vs[b:b + 1, :, :S[b]],
                              np.array([P[b]]))
    return out


@pytest.mark.parametrize("name", ["c0", "c2-blk8", "c3"])
def test_dense_views_equal_dblk_attend(name):
    dev = require_gpu()
    w = WORKLOADS[name]
    note(f"segments dense {name}")
    d = upload(make_inputs(w, parts=("attn",)), dev)
    o1 = torch.empty_like(d["q"])
    dblock.dblk_attend(d["q"], d["kp"], d["vp"], d["kb"], d["vb"], d["ks"], d["vs"],
                       d["prefix_len"], o1)
    o2 = torch.full_like(d["q"], 7.0)
    args = dblock.attend_args(d["q"], dblock.kv_segment(d["kp"], d["vp"], d["prefix_len"]),
                              dblock.kv_segment(d["kb"], d["vb"]),
                              dblock.kv_segment(d["ks"], d["vs"]), o2)
    dblock.dblk_attend_segments(args, device=dev)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("B,H,D,L,P_cap,S_cap,seed", [
    (3, 4, 128, 64, 200, 90, 1),     # few (b, h): the key range is split, last-arriver merge
    (2, 2, 64, 32, 1500, 300, 2),    # long ranges, many splits
    (8, 32, 64, 16, 40, 24, 3),      # B*H = 256: one split per (b, h)
    (2, 3, 128, 128, 100, 50, 4),    # two query tiles per wave
    (8, 16, 128, 64, 1000, 100, 5),  # eight waves on 640-key splits (whole-row loads)
])
def test_fused_qkv_and_head_interleaved_cache(B, H, D, L, P_cap, S_cap, seed):
    dev = require_gpu()
    note(f"segments strided B={B} H={H} D={D} L={L} P_cap={P_cap} S_cap={S_cap}")
    rng = np.random.default_rng(900 + seed)
    qkv = _bits(rng, (B, L, 3, H, D))                 # fused projection: q, k, v of the block
    pre_k = _bits(rng, (B, P_cap, H, D))               # head-interleaved caches [B][T][H][D]
    pre_v = _bits(rng, (B, P_cap, H, D))
    suf_k = _bits(rng, (B, S_cap, H, D))
    suf_v = _bits(rng, (B, S_cap, H, D))
    P = rng.integers(0, P_cap + 1, B).astype(np.int32)
    Lk = rng.integers(L // 2, L + 1, B).astype(np.int32)
    S = rng.integers(0, S_cap + 1, B).astype(np.int32)
    P[0], S[-1] = P_cap, S_cap                          # the extremes are in the draw
    g_qkv = bf16(qkv, dev)
    g = {n: bf16(a, dev) for n, a in (("pk", pre_k), ("pv", pre_v), ("sk", suf_k), ("sv", suf_v))}
    out_buf = torch.full((B, L, 2, H, D), 3.0, dtype=torch.bfloat16, device=dev)
    out = out_buf[:, :, 1]
    hv = lambda t: t.permute(0, 2, 1, 3)                 # [B][T][H][D] -> [B][H][T][D] view
    lens = [torch.from_numpy(x).to(dev) for x in (P, Lk, S)]
    args = dblock.attend_args(
        g_qkv[:, :, 0],
        dblock.kv_segment(hv(g["pk"]), hv(g["pv"]), lens[0]),
        dblock.kv_segment(hv(g_qkv[:, :, 1]), hv(g_qkv[:, :, 2]), lens[1]),
        dblock.kv_segment(hv(g["sk"]), hv(g["sv"]), lens[2]), out)
    dblock.dblk_attend_segments(args, device=dev)
    torch.cuda.synchronize()
    got = bf16_to_np(out.contiguous())
    untouched = out_buf[:, :, 0]
    assert bool((untouched == 3.0).all()), "the call wrote outside the output view"

    f = bf16_bits_to_f64
    tr = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    ref = _oracle_rows(f(qkv[:, :, 0]), tr(f(pre_k)), tr(f(pre_v)), tr(f(qkv[:, :, 1])),
                       tr(f(qkv[:, :, 2])), tr(f(suf_k)), tr(f(suf_v)), P, Lk, S)
    err = attention_row_rel_err(got, ref)
    note(f"  row rel err {err:.2e}; lengths P={P.tolist()} Lk={Lk.tolist()} S={S.tolist()}")
    assert err <= 1e-2


def test_sequences_with_missing_segments():
    """Ragged lengths down to zero: a sequence with only suffix keys, one with
    only prefix keys, one with no key at all (written as zeros)."""
    dev = require_gpu()
    B, H, D, L, P_cap, S_cap = 4, 2, 64, 32, 300, 200
    note("segments with empty rows")
    rng = np.random.default_rng(77)
    q = _bits(rng, (B, L, H, D))
    arr = {n: _bits(rng, (B, H, T, D)) for n, T in (("kp", P_cap), ("vp", P_cap), ("kb", L),
                                                    ("vb", L), ("ks", S_cap), ("vs", S_cap))}
    P = np.array([0, 250, 0, 17], dtype=np.int32)
    Lk = np.array([0, 0, 0, 32], dtype=np.int32)
    S = np.array([150, 0, 0, 199], dtype=np.int32)
    t = {n: bf16(a, dev) for n, a in arr.items()}
    out = torch.full((B, L, H, D), 5.0, dtype=torch.bfloat16, device=dev)
    lens = [torch.from_numpy(x).to(dev) for x in (P, Lk, S)]
    g_q = bf16(q, dev)             # the argument struct holds raw pointers: keep q alive
    args = dblock.attend_args(g_q, dblock.kv_segment(t["kp"], t["vp"], lens[0]),
                              dblock.kv_segment(t["kb"], t["vb"], lens[1]),
                              dblock.kv_segment(t["ks"], t["vs"], lens[2]), out)
    dblock.dblk_attend_segments(args, device=dev)
    torch.cuda.synchronize()
    got = bf16_to_np(out)
    f = bf16_bits_to_f64
    ref = _oracle_rows(f(q), *(f(arr[n]) for n in ("kp", "vp", "kb", "vb", "ks", "vs")), P, Lk, S)
    assert (got[2] == 0).all()                          # no key: zeros
    keep = [0, 1, 3]
    err = attention_row_rel_err(got[keep], ref[keep])
    note(f"  row rel err {err:.2e}")
    assert err <= 1e-2
