"""Writes tests/golden/oracle_regression.json: sampled outputs of the CPU
oracle on a small seeded workload.  Calls only oracle/ (and the seeded input
generator); nothing here comes from the HIP path.

    python tests/golden/make_oracle_regression.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from sparse_mla_amd import workload  # noqa: E402

CASE = dict(name="sparse_b32_l4096_k2048", B=2, L=300, k=64)


def compute():
    w = workload.make(CASE["name"], B=CASE["B"], L=CASE["L"], k=CASE["k"])
    r = oracle.decode(w.q_nope, w.q_pe, w.kv, w.pe, w.wkv_b, w.seq_lens, w.indices, w.scale)
    rng = np.random.default_rng(0)
    picks = [(int(b), int(h), int(d)) for b, h, d in zip(
        rng.integers(0, CASE["B"], 16), rng.integers(0, 128, 16), rng.integers(0, 128, 16))]
    return dict(
        case=CASE,
        out_samples=[[b, h, d, float(r["out"][b, h, d])] for b, h, d in picks],
        lse=r["lse"].tolist(),
        out_abs_max=float(np.max(np.abs(r["out"]))),
    )


if __name__ == "__main__":
    oracle.build(force=False)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", path)
