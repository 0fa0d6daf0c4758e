"""The head-sharded step (the *_heads calls through the C ABI; the binding
passes the head count of its tensors): one GPU's share of 16, 32 or 64 of the
128 heads, with its rows of wkv_b ("Queries" page, init excerpt: wkv_b is a
column-parallel layer, n_local_heads heads per rank).  Outputs against the
oracle on the sliced heads, and bit for bit against the same heads of the
full 128-head step (every head is computed on its own)."""
import numpy as np
import pytest
import torch

from sparse_mla_amd import workload
from tests.gpu_common import (REL_TOL, bf16_query_scores, check_rowsums, f64, gather_rows_for_oracle, oracle_ref,
                              rel_err, slot_rows, to_gpu)

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


def _shard(w, h0, H):
    """The workload restricted to heads h0 .. h0 + H - 1 (views re-made contiguous)."""
    return workload.Workload(spec=w.spec, B=w.B, seq_lens=w.seq_lens, max_len=w.max_len,
                             q_nope=w.q_nope[:, :, h0:h0 + H].contiguous(), q_pe=w.q_pe[:, :, h0:h0 + H].contiguous(),
                             cache=w.cache, wkv_b=w.wkv_b[h0 * 256:(h0 + H) * 256].contiguous(), indices=w.indices,
                             scale=w.scale)


def _step(mla, g, S, fused=True):
    H = g.q_nope.shape[2]
    bufs = mla.DecodeBuffers.allocate(g.B, g.k_max, g.indices is None, num_splits=S, heads=H)
    out = mla.decode_step(bufs, g.q_nope, g.q_pe, g.kv, g.pe, g.wkv_b, g.seq_lens, g.max_len, g.indices, g.scale,
                          fused=fused)
    torch.cuda.synchronize()
    return bufs, out.clone()


CASES = [
    ("sparse_b32_l4096_k2048", 5, 700, 300, 1),
    ("sparse_b32_l4096_k2048", 5, 700, 300, 3),
    ("longctx_b64_k2048", 4, 3000, 700, 2),
    ("dense_p1000_b1", 2, 1001, None, 4),
]


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-B{c[1]}-k{c[3]}-S{c[4]}")
def test_heads_small(mla, H, case):
    name, B, L, k, S = case
    print(f"[heads] H={H} {case}", flush=True)
    w = workload.make(name, B=B, L=L, k=k)
    fusings = (True, False) if S > 1 else (True,)
    full = {}
    for fused in fusings:     # the fused and the separate merge round differently: compare like with like
        fb, fo = _step(mla, to_gpu(w), S, fused)
        full[fused] = (fo, fb.lse.clone())
    for h0 in (0, 128 - H):
        ws = _shard(w, h0, H)
        g = to_gpu(ws)
        for fused in fusings:
            bufs, out = _step(mla, g, S, fused)
            assert torch.equal(out, full[fused][0][:, :, h0:h0 + H])
            assert torch.equal(bufs.lse, full[fused][1][:, h0:h0 + H])
        ref = oracle_ref(ws, want_weights=True)
        assert rel_err(f64(out)[:, 0], ref["out"]) <= REL_TOL
        check_rowsums(ref, f64(bufs.lse), q16_scores=bf16_query_scores(ref, ws.q_pe, slot_rows(ws), ws.scale))


@pytest.mark.parametrize("H", [16, 32, 64])
def test_heads_headline_full_size(mla, H):
    """B = 64, k = 2048 of ragged 2048-32768 positions, in the planned launch:
    each shard equals its heads of the full step; sampled sequences against
    the oracle."""
    name = workload.HEADLINE
    print(f"[heads] full size {name} H={H}", flush=True)
    w = workload.make(name, device="cpu", cache_device="cuda")
    g = workload.Workload(spec=w.spec, B=w.B, seq_lens=w.seq_lens.cuda(), max_len=w.max_len, q_nope=w.q_nope.cuda(),
                          q_pe=w.q_pe.cuda(), cache=w.cache, wkv_b=w.wkv_b.cuda(), indices=w.indices.cuda(),
                          scale=w.scale)
    S = mla.mla_plan(w.B, w.k_max, False)
    _, full_out = _step(mla, g, S)
    h0 = 128 - H
    gs = _shard(g, h0, H)
    _, out = _step(mla, gs, S)
    assert torch.equal(out, full_out[:, :, h0:h0 + H])
    rows = [0, 40]
    kv, pe, klens, kidx = gather_rows_for_oracle(g, rows)
    sel = torch.tensor(rows)
    ref = oracle.decode(w.q_nope[sel][:, :, h0:h0 + H], w.q_pe[sel][:, :, h0:h0 + H], kv, pe,
                        w.wkv_b[h0 * 256:(h0 + H) * 256], klens, kidx, w.scale)
    assert rel_err(f64(out)[rows, 0], ref["out"]) <= REL_TOL
