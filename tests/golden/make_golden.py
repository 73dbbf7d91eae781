"""Writes c1_oracle.json: the oracle's selection and attention output on the tiny fp32 workload
(C1: B1, 2 query heads / 1 KV head, d64, 1024 tokens, 4+4 blocks).

A regression record of the oracle's float64 build (calls only oracle/ and the input generator),
not a pin: the
pins are in tests/test_oracle_pins.py.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from nosa_inputs import WORKLOADS, generate  # noqa: E402
from oracle import oracle as O  # noqa: E402


def main():
    w = WORKLOADS["C1"]
    x = generate(w)
    # the float64 build: the record bounds the default float32 build's rounding as well
    kp = O.pool_keys(x["k"], 32, precision="f64")
    r = O.decode_step(x["q"], kp, x["evict"], x["k"], x["v"], w.n_blocks, w.kq, w.ke, 2, precision="f64")
    rec = {
        "workload": "C1 (seed 1): B1, Hq 2, Hkv 1, d 64, 16 blocks of 64, kq 4, ke 4, fp32",
        "generator": "nosa_inputs.generate(WORKLOADS['C1'])",
        "block_scores": [float(v) for v in r["scores"].reshape(-1)],
        "agn_state": r["agn_state"].reshape(-1).tolist(),
        "selected": r["selected"].reshape(-1).tolist(),
        "out": [float(v) for v in r["out"].reshape(-1)],
    }
    with open(os.path.join(HERE, "c1_oracle.json"), "w") as f:
        json.dump(rec, f, indent=1)


if __name__ == "__main__":
    main()
