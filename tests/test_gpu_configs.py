"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (mla_plan's splits, combine fused into the value-up launch):
on every sequence, outputs within 1e-2 * max|O_ref| (per group of 16
sequences), softmax rows summing to one within 1e-3 (the oracle's exact
scores through the kernel's log-sum-exp) and the attended position set
bit-exact; on sampled sequences also the kernel's own scores and the
oracle's scores with the absorbed query rounded to bf16 through it."""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_amd import workload
from tests.gpu_common import (REL_TOL, attended_sets_equal, bf16_query_scores, check_rowsums, f64,
                              gather_rows_for_oracle, rel_err)

pytestmark = pytest.mark.gpu

SAMPLES = {"dense_p1000_b1": [0], "sparse_b32_l4096_k2048": [0, 17, 31], "longctx_b64_k2048": [0, 33, 63],
           "verylong_b128_l131072_k2048": [0, 64, 127], "dense_fp8w_b64_l8192": [0, 63]}


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


@pytest.mark.parametrize("name", list(workload.SPECS))
def test_full_size(mla, name):
    print(f"[full-size] {name}", flush=True)
    w = workload.make(name, device="cpu", cache_device="cuda")
    dev = "cuda"
    q_nope, q_pe = w.q_nope.to(dev), w.q_pe.to(dev)
    lens = w.seq_lens.to(dev)
    idx = None if w.indices is None else w.indices.to(dev)
    if w.wkv_b_fp8 is not None:
        wkv_b = mla.mla_dequant_wkv_b_fp8(w.wkv_b_fp8.to(dev), w.wkv_b_scale.to(dev))
        bits, _ = oracle.dequant_fp8(w.wkv_b_fp8, w.wkv_b_scale)
        wkv_b_ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        wkv_b = w.wkv_b.to(dev)
        wkv_b_ref = w.wkv_b
    S = mla.mla_plan(w.B, w.k_max, idx is None)
    bufs = mla.DecodeBuffers.allocate(w.B, w.k_max, idx is None, num_splits=S)
    words = (w.max_len + 31) // 32
    bitmap = torch.zeros((w.B, words), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = mla.decode_step(bufs, q_nope, q_pe, w.kv, w.pe, wkv_b, lens, w.max_len, idx, w.scale,
                          flags=mla.MLA_FLAG_VALIDATE, bitmap=bitmap, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    out = out.clone()
    lse_run = bufs.lse.clone()
    # Same plan without validation: bit-identical output.
    out_plain = mla.decode_step(bufs, q_nope, q_pe, w.kv, w.pe, wkv_b, lens, w.max_len, idx, w.scale).clone()
    torch.cuda.synchronize()
    assert torch.equal(out_plain, out)
    # Same plan writing the kernel's own scores: identical output, and its
    # softmax rows (scores through its LSE) sum to one.
    k_max = w.max_len if idx is None else w.k_max
    scores = torch.empty((w.B, 128, k_max), dtype=torch.float32, device=dev)
    out_sc = mla.decode_step(bufs, q_nope, q_pe, w.kv, w.pe, wkv_b, lens, w.max_len, idx, w.scale,
                             flags=mla.MLA_FLAG_WRITE_SCORES, scores=scores)
    torch.cuda.synchronize()
    assert torch.equal(out_sc, out) and torch.equal(bufs.lse, lse_run)

    rows = SAMPLES[name]
    w.cache_dev = w.cache
    gw = w
    gw.seq_lens = lens
    gw.indices = idx
    kv, pe, klens, kidx = gather_rows_for_oracle(gw, rows)
    sel = torch.tensor(rows)
    ref = oracle.decode(w.q_nope[sel], w.q_pe[sel], kv, pe, wkv_b_ref, klens, kidx, w.scale, want_weights=True)
    got = f64(out)[rows, 0]
    assert rel_err(got, ref["out"]) <= REL_TOL
    lse = f64(lse_run)[rows]
    rows_k = [torch.cat([kv[i], pe[i]], -1) for i in range(len(rows))]    # compacted slot order
    q16 = bf16_query_scores(ref, w.q_pe[sel], [r.double().numpy() for r in rows_k], w.scale)
    check_rowsums(ref, lse, f64(scores[sel.to(dev)]), q16, all_exact=True)
    # Every sequence, in groups of 16: outputs against the oracle, and the
    # oracle's scores through the kernel's log-sum-exp summing to one.
    got_all, lse_all = f64(out)[:, 0], f64(lse_run)
    for g0 in range(0, w.B, 16):
        grp = list(range(g0, min(w.B, g0 + 16)))
        kv, pe, klens, kidx = gather_rows_for_oracle(gw, grp)
        sel = torch.tensor(grp)
        r = oracle.decode(w.q_nope[sel], w.q_pe[sel], kv, pe, wkv_b_ref, klens, kidx, w.scale, want_weights=True)
        assert rel_err(got_all[grp], r["out"]) <= REL_TOL, f"sequences {grp[0]} .. {grp[-1]}"
        check_rowsums(r, lse_all[grp], all_exact=True)
    # attended set: bit t of row b <=> t is a selected in-range position, every row
    assert attended_sets_equal(bitmap, w)
