"""The allocation-free decode entry point (mla_sparse_decode_noalloc,
through the C ABI) against the existing one (mla_sparse_decode with a
caller-owned workspace, then mla_combine): identical latent mix and
log-sum-exp, on two calls in a row, the second with a smaller input, and
both within the target tolerance of the oracle; plus its host-side
scratch limit."""
import numpy as np
import pytest
import torch

from sparse_mla_amd import workload
from tests.gpu_common import REL_TOL, bf16_query_scores, check_rowsums, f64, oracle_ref, rel_err, slot_rows, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


def _case(mla, name, B, L, k, S):
    w = workload.make(name, B=B, L=L, k=k)
    g = to_gpu(w)
    q_abs = mla.mla_absorb_q(g.q_nope, g.wkv_b)
    k_max = w.k_max
    # The existing entry point with a workspace, then the separate merge.
    bufs = mla.DecodeBuffers.allocate(w.B, k_max, w.indices is None, num_splits=S)
    mla.mla_sparse_decode(q_abs, g.q_pe, g.kv, g.pe, g.seq_lens, g.max_len, g.indices, g.scale, S,
                          bufs.workspace, bufs.o_latent, bufs.lse, k_max=k_max)
    mla.mla_combine(bufs.workspace, w.B, S, bufs.o_latent, bufs.lse)
    # The allocation-free one into fresh outputs (filled with NaN first).
    o2 = torch.full_like(bufs.o_latent, float("nan"))
    lse2 = torch.full_like(bufs.lse, float("nan"))
    mla.mla_sparse_decode_noalloc(q_abs, g.q_pe, g.kv, g.pe, g.seq_lens, g.max_len, g.indices, g.scale, S, o2,
                                  lse2, k_max=k_max)
    torch.cuda.synchronize()
    return w, bufs, o2, lse2


def test_noalloc_matches_workspace_path_twice(mla):
    print("[noalloc] call 1: B=64 k=2048 S=4; call 2: B=5 k=300 S=3", flush=True)
    for (name, B, L, k, S) in [("longctx_b64_k2048", 64, 4000, 2048, 4), ("sparse_b32_l4096_k2048", 5, 900, 300, 3)]:
        w, bufs, o2, lse2 = _case(mla, name, B, L, k, S)
        assert torch.equal(o2, bufs.o_latent)
        assert torch.equal(lse2, bufs.lse)
        rows = [0, B - 1]
        wr = workload.Workload(spec=w.spec, B=len(rows), seq_lens=w.seq_lens[rows], max_len=w.max_len,
                               q_nope=w.q_nope[rows], q_pe=w.q_pe[rows], cache=w.cache[rows], wkv_b=w.wkv_b,
                               indices=w.indices[rows], scale=w.scale)
        ref = oracle_ref(wr, want_weights=True)
        assert rel_err(f64(o2)[rows], ref["o_lat"]) <= REL_TOL
        check_rowsums(ref, f64(lse2)[rows], q16_scores=bf16_query_scores(ref, wr.q_pe, slot_rows(wr), wr.scale))


def test_noalloc_one_split_and_limit(mla):
    w, bufs, o2, lse2 = _case(mla, "dense_p1000_b1", 2, 1001, None, 1)
    assert torch.equal(o2, bufs.o_latent) and torch.equal(lse2, bufs.lse)
    limit = mla.mla_noalloc_scratch_bytes()
    assert limit == 40 << 20
    # 64 splits of 128 sequences need 64 * 128 * 128 * 1032 bytes > the limit:
    # rejected on the host before anything is enqueued.
    g = to_gpu(workload.make("sparse_b32_l4096_k2048", B=128, L=2048, k=2048))
    q_abs = torch.zeros((128, 128, 512), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q_abs)
    with pytest.raises(mla.MLAError) as ei:
        mla.mla_sparse_decode_noalloc(q_abs, g.q_pe, g.kv, g.pe, g.seq_lens, g.max_len, g.indices, g.scale, 64, o)
    assert ei.value.status == 8
    assert mla.mla_workspace_bytes(128, 64) > limit
