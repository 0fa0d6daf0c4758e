"""GPU parity of the online softmax's lazy rescale (the reference maximum
moved with live accumulators), on inputs with planted score spikes
(tests/rescale_inputs.py): the oracle's scores first show that the rescale
fires, then the decode's latent mix, head outputs and log-sum-exp are
compared with the oracle, in sparse and dense mode, with one split and
several, through the separate combine and the combine fused into the
value-up.  The sparse inputs include a split whose first block is fully
masked ("Softmax" page, formula for A)."""
import pytest
import torch

from tests.gpu_common import REL_TOL, bf16_query_scores, check_rowsums, f64, oracle_ref, rel_err, slot_rows, to_gpu
from tests.rescale_inputs import rescale_events, spike_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


@pytest.mark.parametrize("mode,S", [("sparse", 1), ("sparse", 2), ("sparse", 4), ("dense", 1), ("dense", 4)])
def test_rescale_parity(mla, mode, S):
    print(f"[rescale] mode={mode} S={S}", flush=True)
    w = spike_workload(mode, S)
    ref = oracle_ref(w, want_weights=True)
    events, _ = rescale_events(ref["scores"], S, margin=0.5)
    assert len(events) > 0
    q16 = bf16_query_scores(ref, w.q_pe, slot_rows(w), w.scale)
    g = to_gpu(w)
    k_max = w.k_max
    scores = torch.empty((w.B, 128, k_max), dtype=torch.float32, device="cuda")
    for fused in ((False, True) if S > 1 else (False,)):
        bufs = mla.DecodeBuffers.allocate(w.B, k_max, w.indices is None, num_splits=S)
        out = mla.decode_step(bufs, g.q_nope, g.q_pe, g.kv, g.pe, g.wkv_b, g.seq_lens, g.max_len, g.indices,
                              g.scale, flags=mla.MLA_FLAG_WRITE_SCORES, scores=scores, fused=fused)
        torch.cuda.synchronize()
        if not fused:
            assert rel_err(f64(bufs.o_latent), ref["o_lat"]) <= REL_TOL
        assert rel_err(f64(out)[:, 0], ref["out"]) <= REL_TOL
        check_rowsums(ref, f64(bufs.lse), f64(scores), q16)
