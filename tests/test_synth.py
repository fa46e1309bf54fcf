"""The seeded input generator: determinism, bf16 rounding, recipe statistics."""
import numpy as np
import pytest
import torch

from synth import WORKLOADS, bf16_bits_to_f32, custom_workload, f32_to_bf16_bits, make_inputs
from synth.workloads import CHUNK, _normal_bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30, -3.3895314e38,
                                  1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125: even mantissa (1.0) wins
    assert bf16_bits_to_f32(f32_to_bf16_bits(np.array([1.0 + 2 ** -8], np.float32)))[0] == 1.0
    assert bf16_bits_to_f32(f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], np.float32)))[0] == 1.015625


def test_deterministic_and_chunk_independent():
    w = WORKLOADS["c0"]
    a = make_inputs(w); b = make_inputs(w)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    # spans several chunks; thread scheduling must not matter
    x = _normal_bf16((7, 7), "w", (3, CHUNK + 5))
    y = _normal_bf16((7, 7), "w", (3, CHUNK + 5))
    np.testing.assert_array_equal(x, y)
    assert x[0, :5].tolist() != x[1, :5].tolist()


def test_shapes_and_mask_fixup():
    w = custom_workload("t", 1, B=40, L=16, mask_p=0.01)
    inp = make_inputs(w)
    assert inp["q"].shape == (40, 16, 2, 64) and inp["kp"].shape == (40, 2, 32, 64)
    assert inp["w"].shape == (512, 128) and inp["h"].shape == (640, 128)
    assert (inp["mask"].sum(1) >= 1).all()
    assert (inp["tokens"][inp["mask"] == 1] == w.mask_id).all()
    assert ((inp["tokens"] >= 0) & (inp["tokens"] < w.V)).all()


def test_ragged_prefix_range():
    w = WORKLOADS["c3"]
    # full c3 is large: check the jitter draw only
    from synth.workloads import _rng
    lo, hi, add = w.prefix_jitter
    pl = _rng(w.input_key, "jitter").integers(lo, hi + 1, size=w.B) + add
    assert pl.min() >= 3584 + 768 and pl.max() <= w.P_cap == 4864


def test_registry_shapes():
    c2 = [WORKLOADS[f"c2-blk{i}"] for i in (0, 8, 15)]
    assert [w.S for w in c2] == [960, 448, 0] and all(w.T_cap == 1280 for w in c2)
    assert WORKLOADS["c4-tau70"].input_key == WORKLOADS["c4-tau95"].input_key
    assert WORKLOADS["c1-mask10"].input_key == WORKLOADS["c1-mask100"].input_key
    assert WORKLOADS["c1-mask10"].mask_key != WORKLOADS["c1-mask100"].mask_key


def test_planted_spike_statistics():
    # logit of the planted token is close to a_i: argmax hits t_i for most rows
    w = WORKLOADS["c0"]
    inp = make_inputs(w, parts=("lmhead",))
    h = bf16_bits_to_f32(inp["h"]).astype(np.float64)
    W = bf16_bits_to_f32(inp["w"]).astype(np.float64)
    l = h @ W.T
    rows = np.arange(len(inp["t"]))
    err = np.abs(l[rows, inp["t"]] - inp["a"])
    assert np.median(err) < 1.0
    big = inp["a"] > 15
    assert (l[rows[big]].argmax(1) == inp["t"][big]).mean() > 0.9
