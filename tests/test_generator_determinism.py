"""The seeded input generator is deterministic and draws what its recipe says.

* Every tensor drawn on the CPU for small versions of each workload hashes to
  the SHA-256 stored in ``tests/golden/generator_hashes.json`` (written by
  ``make_generator_hashes.py``, which calls only the generator), and drawing
  twice in one process gives the same bytes.
* Structure: index rows are distinct, in range and -1 padded only where the
  sequence is shorter than k; the "recent" recipe holds its whole recent
  window; ragged lengths stay in [lo, L]; variants draw different tensors.
* On the GPU (``-m gpu``), the tensors drawn with device="cuda" are the same
  bytes on two draws, and the CPU-drawn lengths and index lists match the
  stored hashes after the move.
"""
import json
from pathlib import Path

import pytest
import torch

from sparse_mla_amd import workload
from tests.golden import make_generator_hashes as mgh

GOLD = json.loads((Path(__file__).parent / "golden" / "generator_hashes.json").read_text())["cases"]


def _draws():
    for c in mgh.CASES:
        yield mgh.key("make", *c), lambda c=c: mgh.workload_tensors(*c)
    for c in mgh.PREFILL:
        yield mgh.key("prefill", *c), lambda c=c: mgh.prefill_tensors(*c)
    for B in mgh.OPROJ:
        yield mgh.key("output_proj", B), lambda B=B: mgh.oproj_tensors(B)


DRAWS = list(_draws())


@pytest.mark.parametrize("key,draw", DRAWS, ids=[k for k, _ in DRAWS])
def test_stored_hashes(key, draw):
    got = {n: mgh.digest(t) for n, t in draw().items()}
    assert got == GOLD[key]


@pytest.mark.parametrize("key,draw", DRAWS[:3], ids=[k for k, _ in DRAWS[:3]])
def test_two_draws_identical(key, draw):
    a, b = draw(), draw()
    for n in a:
        if a[n] is None:
            assert b[n] is None
        else:
            assert torch.equal(a[n].view(torch.uint8) if a[n].dtype == torch.bfloat16 else a[n],
                               b[n].view(torch.uint8) if b[n].dtype == torch.bfloat16 else b[n]), n


@pytest.mark.parametrize("name,B,L,k", [("sparse_b32_l4096_k2048", 4, 900, 300),
                                         ("longctx_b64_k2048", 6, 9000, 2048),
                                         ("longctx_b64_k2048", 5, 3000, 300),
                                         ("verylong_b128_l131072_k2048", 2, 3000, 2048)])
def test_index_structure(name, B, L, k):
    w = workload.make(name, B=B, L=L, k=k)
    spec = workload.SPECS[name]
    lens = w.seq_lens.tolist()
    if spec.lens == "ragged":
        assert all(spec.lo <= x <= L for x in lens)
    else:
        assert lens == [L] * B
    for b, Lb in enumerate(lens):
        row = w.indices[b].tolist()
        valid = [i for i in row if i >= 0]
        assert len(valid) == min(Lb, k)
        assert len(set(valid)) == len(valid)
        assert all(0 <= i < Lb for i in valid)
        assert row.count(-1) == k - len(valid)
        if spec.select == "recent" and Lb > k:
            win = min(512, k // 4)
            assert set(range(Lb - win, Lb)) <= set(valid)
            assert min(valid) < Lb - win          # the rest is drawn from the earlier positions
            assert valid[:win] != list(range(Lb - win, Lb))   # shuffled


def test_prefill_index_structure():
    B, T, k = 1, 300, 64
    p = workload.make_prefill(B, T, k)
    for s in range(T):
        row = p.indices[0, s].tolist()
        valid = [i for i in row if i >= 0]
        assert len(valid) == len(set(valid)) == min(k, T)
        assert all(0 <= i < T for i in valid)
        causal = [i for i in valid if i <= s]
        if s + 1 <= k:
            assert sorted(causal) == list(range(s + 1))
        else:
            assert len(causal) == k
            assert set(range(s + 1 - min(512, k // 4), s + 1)) <= set(causal)


def test_variants_differ():
    a = mgh.workload_tensors("sparse_b32_l4096_k2048", 3, 300, 64, 0)
    b = mgh.workload_tensors("sparse_b32_l4096_k2048", 3, 300, 64, 1)
    for n in ("q_nope", "q_pe", "cache", "wkv_b", "indices"):
        assert mgh.digest(a[n])[2] != mgh.digest(b[n])[2], n


@pytest.mark.gpu
def test_cuda_draws_deterministic():
    name, B, L, k = "longctx_b64_k2048", 3, 3000, 700
    a = workload.make(name, device="cuda", B=B, L=L, k=k)
    b = workload.make(name, device="cuda", B=B, L=L, k=k)
    for n in ("q_nope", "q_pe", "cache", "wkv_b", "indices", "seq_lens"):
        assert mgh.digest(getattr(a, n)) == mgh.digest(getattr(b, n)), n
    gold = GOLD[mgh.key("make", name, B, L, k, 0)]
    assert mgh.digest(a.indices) == gold["indices"]
    assert mgh.digest(a.seq_lens) == gold["seq_lens"]
