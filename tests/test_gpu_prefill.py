"""GPU parity of the sparse prefill (mla_sparse_prefill, through the C ABI)
against the prefill oracle ("Queries" page, prefill mode: the full-sequence
MHA form with the index and causal masks): head outputs within
1e-2 * max |O_ref|, the attended set of every query token bit-exact, and
softmax row sums against the oracle's scores (taken from the decode oracle
on each token's causal prefix, which the prefill oracle's pins tie to it).
At full size (T = 4096) the outputs and row sums are checked on every 16th
token and a set of edge tokens."""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_amd import workload
from tests.gpu_common import REL_TOL, bf16_query_scores, check_rowsums, f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


def _run(mla, p, S=None):
    dev = "cuda"
    T = p.T
    idx = None if p.indices is None else p.indices.to(dev)
    words = (T + 31) // 32
    bitmap = torch.zeros((p.B * T, words), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    lse = torch.empty((p.B * T, 128), dtype=torch.float32, device=dev)
    cache = p.cache.to(dev)
    out = mla.mla_sparse_prefill(p.q_nope.to(dev), p.q_pe.to(dev), cache[..., :512], cache[..., 512:],
                                 p.wkv_b.to(dev), idx, p.scale, num_splits=S, lse=lse,
                                 flags=mla.MLA_FLAG_VALIDATE, bitmap=bitmap, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, lse, bitmap


def _bits(bitmap, T):
    b = bitmap.cpu().numpy().view(np.uint32)
    return np.unpackbits(b.view(np.uint8), axis=1, bitorder="little")[:, :T]


def _row_refs(p, rows):
    """Decode-oracle results for prompt rows [(b, s)], each over positions
    0 .. s with the token's index row (later positions dropped), with its
    per-slot scores and weights; plus the bf16-query scores."""
    refs, q16 = [], []
    cache = p.cache.cpu()
    for (b, s) in rows:
        if p.indices is None:
            row = np.concatenate([np.arange(s + 1), np.full(p.T - s - 1, -1)])
        else:
            row = p.indices[b, s].cpu().numpy().astype(np.int64)
            row = np.where(row <= s, row, -1)
        r = oracle.decode(p.q_nope[b:b + 1, s], p.q_pe[b:b + 1, s], cache[b:b + 1, :s + 1, :512],
                          cache[b:b + 1, :s + 1, 512:], p.wkv_b, np.array([s + 1], dtype=np.int32), row[None],
                          p.scale, want_weights=True)
        pos = np.where(row >= 0, row, 0)
        q16.append(bf16_query_scores(r, p.q_pe[b:b + 1, s], [cache[b, pos].double().numpy()], p.scale)[0])
        refs.append(r)
    keys = ("out", "lse", "scores", "weights")
    ref = {k: np.concatenate([r[k] for r in refs]) for k in keys}
    return ref, np.stack(q16)


def _row_refs_compact(p, rows):
    """Decode-oracle results for many prompt rows [(b, s)] in one call, each
    over the positions its index row selects at or before s (in slot order),
    moved to the front of a per-row cache; with per-slot scores and weights."""
    cache = p.cache.cpu()
    sel, lens = [], []
    for (b, s) in rows:
        if p.indices is None:
            pos = np.arange(s + 1)
        else:
            r = p.indices[b, s].cpu().numpy().astype(np.int64)
            pos = r[(r >= 0) & (r <= s)]
        sel.append(cache[b, torch.from_numpy(pos)])
        lens.append(len(pos))
    n, k = len(rows), max(lens)
    kv = torch.zeros((n, k, 512), dtype=torch.bfloat16)
    pe = torch.zeros((n, k, 64), dtype=torch.bfloat16)
    idx = np.full((n, k), -1, dtype=np.int64)
    for i, r in enumerate(sel):
        kv[i, : lens[i]] = r[:, :512]
        pe[i, : lens[i]] = r[:, 512:]
        idx[i, : lens[i]] = np.arange(lens[i])
    qn = torch.stack([p.q_nope[b, s] for (b, s) in rows])
    qp = torch.stack([p.q_pe[b, s] for (b, s) in rows])
    return oracle.decode(qn, qp, kv, pe, p.wkv_b, np.array(lens, dtype=np.int32), idx, p.scale,
                         want_weights=True)


@pytest.mark.parametrize("k,S", [(48, None), (48, 1), (48, 3), (None, None)])
def test_prefill_small(mla, k, S):
    print(f"[prefill] B=2 T=200 k={k} S={S}", flush=True)
    p = workload.make_prefill(2, 200, k)
    out, lse, bitmap = _run(mla, p, S)
    ref = oracle.prefill(p.q_nope, p.q_pe, p.kv, p.pe, p.wkv_b, p.indices, p.scale, want_attended=True)
    assert rel_err(f64(out), ref["out"]) <= REL_TOL
    assert np.array_equal(_bits(bitmap, p.T), ref["attended"].reshape(p.B * p.T, p.T))
    rows = [(b, s) for b in range(2) for s in (0, 1, 47, 48, 120, 199)]
    rr, q16 = _row_refs(p, rows)
    sel = [b * p.T + s for (b, s) in rows]
    assert np.allclose(rr["out"], ref["out"].reshape(-1, 128, 128)[sel], rtol=0, atol=1e-12)
    check_rowsums(rr, f64(lse)[sel], q16_scores=q16)


def test_prefill_full_size(mla):
    B, T, k = workload.PREFILL_HEADLINE["B"], workload.PREFILL_HEADLINE["T"], workload.PREFILL_HEADLINE["k"]
    print(f"[prefill] full size B={B} T={T} k={k}", flush=True)
    p = workload.make_prefill(B, T, k)
    out, lse, bitmap = _run(mla, p)
    # attended set of every token: its index row cut at its own position
    got = _bits(bitmap, T)
    idx = p.indices.cpu().numpy()
    for b in range(B):
        for s in range(T):
            r = idx[b, s]
            want = np.zeros(T, dtype=np.uint8)
            want[np.unique(r[(r >= 0) & (r <= s)])] = 1
            assert np.array_equal(got[b * T + s], want), (b, s)
    rows = [(0, s) for s in (0, 1, 511, 2046, 2047, 2048, 3000, 4095)]
    rr, q16 = _row_refs(p, rows)
    sel = [b * T + s for (b, s) in rows]
    got, lse_all = f64(out).reshape(-1, 128, 128), f64(lse)
    assert rel_err(got[sel], rr["out"]) <= REL_TOL
    check_rowsums(rr, lse_all[sel], q16_scores=q16)
    # Every 16th token of the prompt, 64 per oracle call: outputs and the
    # oracle-score row sums through the kernel's log-sum-exp.
    more = [(b, s) for b in range(B) for s in range(0, T, 16)]
    for c0 in range(0, len(more), 64):
        part = more[c0:c0 + 64]
        rr = _row_refs_compact(p, part)
        sel = [b * T + s for (b, s) in part]
        assert rel_err(got[sel], rr["out"]) <= REL_TOL, f"tokens {part[0]} .. {part[-1]}"
        check_rowsums(rr, lse_all[sel])
