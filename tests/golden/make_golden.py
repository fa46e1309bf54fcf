"""Writes oracle_c0.json from the oracle alone (tiny workload c0).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import iteration  # noqa: E402
from synth import WORKLOADS, make_inputs  # noqa: E402


def main():
    w = WORKLOADS["c0"]
    r = iteration(make_inputs(w), w.tau)
    out = {
        "source": "fp64 oracle on workload c0 (tests/golden/make_golden.py)",
        "conf": r["conf"].tolist(),
        "argmax": r["argmax"].tolist(),
        "tokens": r["tokens"].tolist(),
        "mask": r["mask"].tolist(),
        "n": r["n"].tolist(),
        "o_every_97th": r["o"].reshape(-1)[::97].tolist(),
    }
    with open(os.path.join(HERE, "oracle_c0.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()
