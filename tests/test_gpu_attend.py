"""dblk_attend vs the fp64 oracle on sizes the oracle finishes in seconds.

Covers both head dims, every block length class (one or two query tiles per
wave), empty prefix or suffix, key counts that are not multiples of the
64-key tile, one and several key splits, short and long key ranges per split
(one or two waves per query tile), ragged per-sequence prefixes and an
explicit score scale.

Bar: per output row (b, l, h), max-abs error over max-abs reference <= 1e-2.
"""
import numpy as np
import pytest
import torch

from block_wise_decoding_amd import dblock
from oracle import attend, attention_row_rel_err, bf16_bits_to_f64
from synth import custom_workload, make_inputs
from tests.gpu_util import bf16_to_np, note, require_gpu, run_attend, upload

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _oracle(inp, scale=None):
    f = {k: bf16_bits_to_f64(inp[k]) for k in ("q", "kp", "vp", "kb", "vb", "ks", "vs")}
    return attend(f["q"], f["kp"], f["vp"], f["kb"], f["vb"], f["ks"], f["vs"], inp["prefix_len"], scale)


@pytest.mark.parametrize("B,H,D,L,P,S,jitter", [
    (1, 4, 64, 32, 128, 64, None),          # the tiny workload's attention
    (1, 2, 128, 64, 0, 0, None),            # block only
    (2, 3, 128, 16, 100, 0, None),          # no suffix, T not a tile multiple
    (1, 2, 64, 128, 0, 77, None),           # no prefix, two query tiles per wave
    (2, 16, 128, 64, 768, 448, None),       # LLaDA-MoE block 8 shape at B=2
    (3, 2, 128, 48, 300, 33, (10, 300, 0)), # ragged prefixes, 3 query tiles
    (4, 1, 64, 64, 5000, 120, (0, 5000, 0)),  # long, ragged down to an empty prefix
    (1, 8, 128, 64, 4500, 100, (3000, 4500, 0)),  # long ragged cache, few (b, h): many splits
    (1, 16, 128, 64, 768, 448, None),       # LLaDA-MoE block 8 shape (10 splits of 128 keys)
    (2, 1, 128, 16, 4000, 96, (1, 4000, 0)),  # one query tile, ragged down to one prefix key
    (40, 8, 128, 128, 64, 64, None),        # many (b, h): single split path
    # long key ranges (>= 512 keys per split, one query tile per wave): two
    # waves per query tile on the two halves of every key tile
    (16, 16, 128, 64, 600, 40, None),       # one split of 704 keys per (b, h)
    (8, 16, 64, 32, 1000, 50, (200, 1000, 0)),  # two splits, ragged, half the waves idle
    (4, 64, 128, 16, 700, 0, None),         # last tile's second half wholly past the range
    (1, 1, 128, 64, 60000, 5000, None),     # near the 65536-key limit: 255 splits, merged 16 at a time
])
def test_attend_small(B, H, D, L, P, S, jitter):
    dev = require_gpu()
    note(f"attend B={B} H={H} D={D} L={L} P={P} S={S} jitter={jitter}")
    w = custom_workload(f"at{B}_{H}_{D}_{L}_{P}_{S}", B * 7 + H + D + L + P + S,
                        B=B, H=H, D=D, L=L, P_cap=P, S=S, prefix_jitter=jitter)
    inp = make_inputs(w, parts=("attn",))
    o = bf16_to_np(run_attend(upload(inp, dev)))
    ref = _oracle(inp)
    err = attention_row_rel_err(o, ref)
    nsplit_ws = dblock.attend_workspace_size(B, H, L, D, P, S)
    note(f"  row-rel err={err:.2e} (split workspace {nsplit_ws} B)")
    assert err <= TOL


def test_explicit_scale_and_determinism():
    dev = require_gpu()
    w = custom_workload("atscale", 5, B=1, H=2, D=128, L=64, P_cap=200, S=50)
    inp = make_inputs(w, parts=("attn",))
    d = upload(inp, dev)
    o1 = run_attend(d, scale=0.05)
    o2 = run_attend(d, scale=0.05)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    err = attention_row_rel_err(bf16_to_np(o1), _oracle(inp, scale=0.05))
    note(f"scale 0.05: err={err:.2e}")
    assert err <= TOL


def test_out_of_range_prefix_lengths_are_clamped():
    dev = require_gpu()
    w = custom_workload("atclamp", 6, B=3, H=2, D=64, L=32, P_cap=90, S=10)
    inp = make_inputs(w, parts=("attn",))
    d = upload(inp, dev)
    d["prefix_len"] = torch.tensor([-5, 1000, 40], dtype=torch.int32, device=dev)
    o = bf16_to_np(run_attend(d))
    inp2 = dict(inp); inp2["prefix_len"] = np.array([0, 90, 40])
    assert attention_row_rel_err(o, _oracle(inp2)) <= TOL


@pytest.mark.parametrize("vscale", [3.0e4, 1.0e-30, 1.0])
def test_split_partials_keep_extreme_value_ranges(vscale):
    """The split partials travel as fp16 scaled per row by a power of two: V
    values around 3e4 (an unscaled fp16 partial sum over a split would pass
    65504) and around 1e-30 (far below fp16's range) must merge as accurately
    as values of order one.  LLaDA-MoE block 8 shape, ten splits of 128 keys."""
    dev = require_gpu()
    note(f"attend split partials, V scaled by {vscale:g}")
    w = custom_workload("atvscale", 8, B=1, H=4, D=128, L=64, P_cap=768, S=448)
    inp = make_inputs(w, parts=("attn",))
    from synth.workloads import bf16_bits_to_f32, f32_to_bf16_bits
    for k in ("vp", "vb", "vs"):
        inp[k] = f32_to_bf16_bits(bf16_bits_to_f32(inp[k]) * np.float32(vscale))
    assert dblock.attend_workspace_size(1, 4, 64, 128, 768, 448) > 0      # split path
    o = bf16_to_np(run_attend(upload(inp, dev)))
    ref = _oracle(inp)
    assert np.isfinite(o).all()
    err = attention_row_rel_err(o, ref)
    note(f"  row-rel err={err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("B,H,L,P,S", [
    (8, 16, 128, 600, 200),    # two query tiles per wave (the throughput batch's kernel), 8-tile splits
    (4, 8, 64, 4400, 200),     # eight waves on 640-key splits (the long-context kernel)
])
def test_rising_scores_move_the_reference(B, H, L, P, S):
    """The long-range kernels let the softmax reference lag the running max by
    up to 2^8 and move it only past that.  Keys scaled up along the walk (x1
    to x12 from first to last key) make the max climb through many tiles, so
    the reference moves repeatedly, lags in between, and the partial sums
    reach the 2^8 bound; the result must still match the oracle."""
    dev = require_gpu()
    note(f"attend rising scores B={B} H={H} L={L} P={P} S={S}")
    w = custom_workload(f"atrise{B}_{H}_{L}", 31 + B + L, B=B, H=H, D=128, L=L, P_cap=P, S=S)
    inp = make_inputs(w, parts=("attn",))
    from synth.workloads import bf16_bits_to_f32, f32_to_bf16_bits
    T = P + L + S
    for k, off, n in (("kp", 0, P), ("kb", P, L), ("ks", P + L, S)):
        ramp = (1.0 + 11.0 * (off + np.arange(n)) / (T - 1)).astype(np.float32)
        inp[k] = f32_to_bf16_bits(bf16_bits_to_f32(inp[k]) * ramp[None, None, :, None])
    o = bf16_to_np(run_attend(upload(inp, dev)))
    err = attention_row_rel_err(o, _oracle(inp))
    note(f"  row-rel err={err:.2e}")
    assert np.isfinite(o).all()
    assert err <= TOL
