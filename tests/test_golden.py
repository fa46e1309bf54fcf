"""Fixtures under tests/golden/.

* ``dinfer_usage_defaults.json`` holds the constants the dInfer README's usage
  example passes (threshold, mask/eos ids, generation and block length); the
  LLaDA-MoE-shaped workloads must agree with them.
* ``oracle_c0.json`` is written by ``tests/golden/make_golden.py`` (which calls
  only the oracle and the input generator) and guards the oracle against
  unintended changes of its arithmetic.
"""
import json
import os

import numpy as np

from synth import WORKLOADS, make_inputs

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_llada_moe_workloads_follow_usage_defaults():
    g = json.load(open(os.path.join(HERE, "dinfer_usage_defaults.json")))
    for name in ("c2-blk0", "c2-blk8", "c2-blk15"):
        w = WORKLOADS[name]
        assert w.tau == g["threshold"] and w.L == g["block_length"]
        assert w.mask_id == g["mask_id"] and g["eos_id"] < w.V and g["mask_id"] < w.V
        # prefix + block + suffix spans the prompt plus gen_length
        assert w.P_cap + w.L + w.S == 256 + g["gen_length"]
    assert g["gen_length"] // g["block_length"] == 16        # block indices 0..15


def test_oracle_regression_c0():
    from oracle import iteration
    g = json.load(open(os.path.join(HERE, "oracle_c0.json")))
    w = WORKLOADS["c0"]
    r = iteration(make_inputs(w), w.tau)
    np.testing.assert_allclose(r["conf"], g["conf"], rtol=1e-12)
    assert r["argmax"].tolist() == g["argmax"]
    assert r["tokens"].tolist() == g["tokens"] and r["mask"].tolist() == g["mask"]
    np.testing.assert_allclose(r["o"].reshape(-1)[:: 97], g["o_every_97th"], rtol=1e-12, atol=1e-15)
