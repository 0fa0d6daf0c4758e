"""Writes tests/golden/generator_hashes.json: the SHA-256 of every tensor the
seeded input generator draws on the CPU for small versions of each workload
(and of the prefill and output-projection inputs), so that a change in what
the generator draws -- a seed, a distribution, a torch RNG change -- fails a
test instead of silently changing every input.  Calls only the generator.

    python tests/golden/make_generator_hashes.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

from sparse_mla_amd import workload  # noqa: E402

# (name, B, L, k, variant): small enough to draw in well under a second each.
CASES = [
    ("dense_p1000_b1", 1, 1001, None, 0),
    ("sparse_b32_l4096_k2048", 3, 300, 64, 0),
    ("sparse_b32_l4096_k2048", 3, 300, 64, 1),
    ("longctx_b64_k2048", 3, 3000, 700, 0),
    ("longctx_b64_k2048", 4, 40000, 2048, 0),
    ("verylong_b128_l131072_k2048", 2, 5000, 2048, 0),
    ("dense_fp8w_b64_l8192", 2, 200, None, 0),
]
PREFILL = [(2, 100, 48), (1, 64, None)]
OPROJ = [3]


def digest(t):
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    raw = t.view(torch.uint8) if t.dtype != torch.uint8 else t
    h = hashlib.sha256(raw.numpy().tobytes()).hexdigest()
    return [list(t.shape), str(t.dtype).replace("torch.", ""), h]


def workload_tensors(name, B, L, k, variant):
    w = workload.make(name, B=B, L=L, k=k, variant=variant)
    return dict(q_nope=w.q_nope, q_pe=w.q_pe, cache=w.cache, wkv_b=w.wkv_b, indices=w.indices,
                seq_lens=w.seq_lens, wkv_b_fp8=w.wkv_b_fp8, wkv_b_scale=w.wkv_b_scale)


def prefill_tensors(B, T, k):
    p = workload.make_prefill(B, T, k)
    return dict(q_nope=p.q_nope, q_pe=p.q_pe, cache=p.cache, wkv_b=p.wkv_b, indices=p.indices)


def oproj_tensors(B):
    x, wo = workload.output_proj_inputs(B)
    return dict(x=x, wo=wo)


def key(*parts):
    return "/".join("None" if p is None else str(p) for p in parts)


def compute():
    out = {}
    for c in CASES:
        out[key("make", *c)] = {n: digest(t) for n, t in workload_tensors(*c).items()}
    for c in PREFILL:
        out[key("prefill", *c)] = {n: digest(t) for n, t in prefill_tensors(*c).items()}
    for B in OPROJ:
        out[key("output_proj", B)] = {n: digest(t) for n, t in oproj_tensors(B).items()}
    return dict(torch_version=torch.__version__.split("+")[0], cases=out)


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "generator_hashes.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1, sort_keys=True)
