"""GPU parity of every HIP kernel against the CPU oracle on small seeded
inputs that span several tiles and a ragged tail (called through the C ABI
via sparse_mla_amd.binding)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_amd import workload
from tests.gpu_common import (REL_TOL, attended_sets_equal, bf16_query_scores, check_rowsums, f64, oracle_ref,
                              rel_err, slot_rows, to_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


def test_absorb_q(mla):
    w = workload.make("sparse_b32_l4096_k2048", B=37, L=8, k=4)   # two batch tiles, ragged
    g = to_gpu(w)
    q_abs = mla.mla_absorb_q(g.q_nope, g.wkv_b)
    torch.cuda.synchronize()
    ref = oracle.absorb(w.q_nope, w.wkv_b)
    assert rel_err(f64(q_abs), ref) <= 4e-3


@pytest.mark.parametrize("B", [200, 300])
def test_absorb_q_many_batch_tiles(mla, B):
    """More than four 32-row batch tiles: the query rows are staged in groups
    of at most four tiles, each group's tiles requested while the group
    before it is computed, into two alternating tile sets (B = 200: groups
    of 4 and 3; B = 300: 4, 4 and 2, the third reusing the first set)."""
    w = workload.make("sparse_b32_l4096_k2048", B=B, L=8, k=4)
    g = to_gpu(w)
    q_abs = mla.mla_absorb_q(g.q_nope, g.wkv_b)
    torch.cuda.synchronize()
    assert rel_err(f64(q_abs), oracle.absorb(w.q_nope, w.wkv_b)) <= 4e-3


def test_absorb_q_strided_query(mla):
    """q_nope as the first 128 columns of a [B,1,128,192] query tensor."""
    B = 5
    q = torch.randn((B, 1, 128, 192), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    w = workload.make("sparse_b32_l4096_k2048", B=1, L=8, k=4)
    q_abs = mla.mla_absorb_q(q.cuda()[..., :128], w.wkv_b.cuda())
    torch.cuda.synchronize()
    assert rel_err(f64(q_abs), oracle.absorb(q[..., :128], w.wkv_b)) <= 4e-3


def test_value_up(mla):
    B = 45
    gen = torch.Generator().manual_seed(11)
    o_lat = torch.randn((B, 128, 512), generator=gen).to(torch.bfloat16)
    w = workload.make("sparse_b32_l4096_k2048", B=1, L=8, k=4)
    out = mla.mla_value_up(o_lat.cuda(), w.wkv_b.cuda())
    torch.cuda.synchronize()
    assert rel_err(f64(out)[:, 0], oracle.value_up(o_lat, w.wkv_b)) <= 4e-3


def _run_decode(mla, g, S, layout="packed", flags=0, bitmap=None, scores=None, status=None, fused=False):
    B = g.B
    k_max = g.k_max
    bufs = mla.DecodeBuffers.allocate(B, k_max, g.indices is None, num_splits=S)
    if layout == "packed":
        kv, pe = g.kv, g.pe
    else:  # two buffers, as in the pages' code
        kv, pe = g.kv.contiguous(), g.pe.contiguous()
    out = mla.decode_step(bufs, g.q_nope, g.q_pe, kv, pe, g.wkv_b, g.seq_lens, g.max_len, g.indices,
                          g.scale, flags=flags, bitmap=bitmap, scores=scores, status=status, fused=fused)
    torch.cuda.synchronize()
    return bufs, out


CASES = [
    # (name, B, L, k, S, layout)
    ("sparse_b32_l4096_k2048", 3, 300, 100, 1, "packed"),
    ("sparse_b32_l4096_k2048", 3, 300, 100, 3, "packed"),
    ("sparse_b32_l4096_k2048", 3, 300, 100, 2, "split"),
    ("sparse_b32_l4096_k2048", 9, 300, 100, 2, "packed"),   # B * S not a multiple of 8
    ("sparse_b32_l4096_k2048", 3, 300, 64, 3, "packed"),    # split 2 holds no slot
    ("longctx_b64_k2048", 4, 3000, 700, 1, "packed"),
    ("longctx_b64_k2048", 4, 3000, 700, 2, "split"),
    ("longctx_b64_k2048", 4, 3000, 700, 5, "packed"),
    ("dense_p1000_b1", 2, 1001, None, 1, "packed"),
    ("dense_p1000_b1", 2, 1001, None, 4, "split"),
    ("sparse_b32_l4096_k2048", 5, 300, 101, 2, "packed"),   # odd slot count: per-slot range checks
    ("sparse_b32_l4096_k2048", 300, 120, 40, 1, "packed"),  # more workgroups than CUs
    ("dense_p1000_b1", 1, 1001, None, 32, "packed"),          # one row, 32 splits in one value-up pass
    ("dense_p1000_b1", 3, 1001, None, 24, "split"),           # 3 rows, 24 splits (8 empty), two passes
    ("sparse_b32_l4096_k2048", 2, 4096, 2048, 64, "packed"),  # the most splits: one block each
    ("sparse_b32_l4096_k2048", 33, 300, 100, 2, "packed"),    # 32-row value-up tiles, a 1-row tile
    ("sparse_b32_l4096_k2048", 2, 4096, 2048, 1, "packed"),   # one split of 2048 slots: the whole index region
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-B{c[1]}-L{c[2]}-k{c[3]}-S{c[4]}-{c[5]}")
def test_decode_small(mla, case):
    name, B, L, k, S, layout = case
    w = workload.make(name, B=B, L=L, k=k)
    if w.indices is not None:
        w.indices[0, -7:] = -1          # padding slots in one row
    g = to_gpu(w)
    k_max = w.max_len if w.indices is None else w.k_max
    scores = torch.empty((w.B, 128, k_max), dtype=torch.float32, device="cuda")
    bufs, out = _run_decode(mla, g, S, layout, flags=mla.MLA_FLAG_WRITE_SCORES, scores=scores)
    ref = oracle_ref(w, want_weights=True)
    q16 = bf16_query_scores(ref, w.q_pe, slot_rows(w), w.scale)
    assert rel_err(f64(bufs.o_latent), ref["o_lat"]) <= REL_TOL
    assert rel_err(f64(out)[:, 0], ref["out"]) <= REL_TOL
    check_rowsums(ref, f64(bufs.lse), f64(scores), q16)
    if S > 1:  # combine fused into the value-up launch
        bufs.lse.fill_(float("nan"))
        bufs2, out2 = _run_decode(mla, g, S, layout, flags=mla.MLA_FLAG_WRITE_SCORES, scores=scores,
                                  fused=True)
        assert rel_err(f64(out2)[:, 0], ref["out"]) <= REL_TOL
        check_rowsums(ref, f64(bufs2.lse), f64(scores), q16)


def test_decode_strided_q_pe(mla):
    """q_pe as the last 64 columns of a [B,1,128,192] query tensor (head
    stride 192): the query tile staging reads it through its strides."""
    w = workload.make("longctx_b64_k2048", B=3, L=3000, k=300)
    g = to_gpu(w)
    q = torch.zeros((w.B, 1, 128, 192), dtype=torch.bfloat16, device="cuda")
    q[..., 128:] = g.q_pe
    g.q_pe = q[..., 128:]
    assert g.q_pe.stride(2) == 192
    for S in (1, 2):
        bufs, out = _run_decode(mla, g, S)
        ref = oracle_ref(w)
        assert rel_err(f64(out)[:, 0], ref["out"]) <= REL_TOL


def test_decode_validate_bitmap_and_scores(mla):
    """VALIDATE: the attended bitmap equals the oracle's set bit for bit;
    WRITE_SCORES: the kernel's own scores normalise against its LSE."""
    w = workload.make("longctx_b64_k2048", B=3, L=2500, k=300)
    w.indices[1, 10:20] = -1
    g = to_gpu(w)
    words = (w.max_len + 31) // 32
    bitmap = torch.zeros((w.B, words), dtype=torch.int32, device="cuda")
    scores = torch.empty((w.B, 128, w.k_max), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs, out = _run_decode(mla, g, 2, flags=mla.MLA_FLAG_VALIDATE | mla.MLA_FLAG_WRITE_SCORES,
                            bitmap=bitmap, scores=scores, status=status)
    assert int(status.item()) == 0
    ref = oracle_ref(w, want_weights=True)
    bits = bitmap.cpu().numpy().view(np.uint32)
    got = np.zeros((w.B, words * 32), dtype=np.uint8)
    for t in range(32):
        got[:, t::32] = (bits >> t) & 1
    att = ref["attended"]
    n = min(att.shape[1], got.shape[1])
    assert np.array_equal(got[:, :n], att[:, :n])
    assert not got[:, n:].any() and not att[:, n:].any()
    sc = f64(scores)
    ref_sc = ref["scores"]
    masked = np.isneginf(ref_sc)
    assert np.array_equal(np.isneginf(sc), masked)
    assert np.max(np.abs(sc[~masked] - ref_sc[~masked])) <= 2e-2
    check_rowsums(ref, f64(bufs.lse), sc, bf16_query_scores(ref, w.q_pe, slot_rows(w), w.scale))
    assert attended_sets_equal(bitmap, w)


@pytest.mark.parametrize("S,fused", [(1, False), (2, False), (2, True)])
def test_decode_validate_errors(mla, S, fused):
    """Out-of-range and repeated indices and an empty row set the status
    bits; the empty sequence yields NaN and the others stay finite."""
    w = workload.make("sparse_b32_l4096_k2048", B=3, L=200, k=64)
    w.indices[0, 3] = 500            # out of range (L = 200)
    w.indices[1, 5] = w.indices[1, 6]  # duplicate
    w.indices[2, :] = -1             # empty selection
    g = to_gpu(w)
    bitmap = torch.zeros((w.B, 8), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs, out = _run_decode(mla, g, S, flags=mla.MLA_FLAG_VALIDATE, bitmap=bitmap, status=status,
                            fused=fused)
    st = int(status.item())
    assert st == (mla.MLA_DEV_INDEX_OUT_OF_RANGE | mla.MLA_DEV_DUPLICATE_INDEX | mla.MLA_DEV_EMPTY_SELECTION)
    o = f64(out)
    assert np.all(np.isnan(o[2])) and np.all(np.isfinite(o[:2]))
    assert np.all(np.isneginf(f64(bufs.lse)[2]))


def test_dequant_fp8_bit_exact(mla):
    codes, scales = workload.fp8_weights(128 * 256, 512, seed=5000)
    bits, _ = oracle.dequant_fp8(codes, scales)
    out = mla.mla_dequant_wkv_b_fp8(codes.cuda(), scales.cuda())
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, bits)


def test_decode_deterministic_and_order_invariant(mla):
    w = workload.make("sparse_b32_l4096_k2048", B=4, L=1000, k=256)
    g = to_gpu(w)
    _, out1 = _run_decode(mla, g, 2)
    o1 = out1.clone()
    _, out2 = _run_decode(mla, g, 2)
    assert torch.equal(o1, out2)
    perm = torch.randperm(w.k_max, generator=torch.Generator().manual_seed(3))
    g.indices = g.indices[:, perm.cuda()].contiguous()
    _, out3 = _run_decode(mla, g, 2)
    ref = oracle_ref(w)
    assert rel_err(f64(out3)[:, 0], ref["out"]) <= REL_TOL


def _split_chunk(k_max, S):
    c = -(-k_max // S)
    return -(-c // 32) * 32


@pytest.mark.parametrize("L,k,S", [(300, 200, 1), (300, 200, 3), (3000, 1900, 1)])
def test_decode_masked_slots_compacted(mla, L, k, S):
    """Slots that select nothing (-1 padding, a negative value, values past
    the sequence) scattered through every row, and with several splits one
    split of a row holding none at all: unless per-slot scores are requested
    the kernel moves each split's valid slots to its front and walks only
    their blocks.  O~, O and the LSE match the oracle on the same selection
    (invalid slots given to it as -1), the row sums hold, the attended bitmap
    and the out-of-range status are exact, and the result equals the
    slot-order path (per-slot scores requested) up to rounding."""
    w = workload.make("sparse_b32_l4096_k2048", B=5, L=L, k=k)
    gen = torch.Generator().manual_seed(41)
    idx = w.indices.clone()
    idx[torch.rand(idx.shape, generator=gen) < 0.5] = -1
    past = (torch.rand(idx.shape, generator=gen) < 0.05) & (idx == -1)
    idx[past] = 100000                      # past every length: masked, flagged
    idx[0, 10] = -7                         # negative and not -1: masked, flagged
    if S > 1:
        idx[2, :_split_chunk(k, S)] = -1     # split 0 of row 2 selects nothing
    clean = idx.clone()
    clean[(clean < 0) | (clean >= L)] = -1
    w.indices = idx
    g = to_gpu(w)
    words = (w.max_len + 31) // 32
    bitmap = torch.zeros((w.B, words), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs, out = _run_decode(mla, g, S, flags=mla.MLA_FLAG_VALIDATE, bitmap=bitmap, status=status)
    o_lat, lse = f64(bufs.o_latent), f64(bufs.lse)
    scores = torch.empty((w.B, 128, w.k_max), dtype=torch.float32, device="cuda")
    bufs2, out2 = _run_decode(mla, g, S, flags=mla.MLA_FLAG_WRITE_SCORES, scores=scores)
    assert int(status.item()) == mla.MLA_DEV_INDEX_OUT_OF_RANGE
    w.indices = clean
    ref = oracle_ref(w, want_weights=True)
    assert rel_err(o_lat, ref["o_lat"]) <= REL_TOL
    assert rel_err(f64(out)[:, 0], ref["out"]) <= REL_TOL
    check_rowsums(ref, lse, None, bf16_query_scores(ref, w.q_pe, slot_rows(w), w.scale))
    assert attended_sets_equal(bitmap, w)
    # Two kernels' bf16 results from differently ordered fp32 sums: a rounding apart.
    assert rel_err(f64(out), f64(out2)) <= 2 * 2.0 ** -8
    assert np.max(np.abs(lse - f64(bufs2.lse))) <= 1e-4


@pytest.mark.parametrize("S", [1, 4])
def test_decode_dense_ragged_stops_at_length(mla, S):
    """Dense selection with ragged lengths: unless per-slot scores are
    requested a split stops at L_b (splits past it are empty) and the result
    matches the oracle."""
    w = workload.make("dense_p1000_b1", B=3, L=1001)
    w.seq_lens = torch.tensor([1001, 300, 37], dtype=torch.int32)
    g = to_gpu(w)
    bufs, out = _run_decode(mla, g, S)
    ref = oracle_ref(w, want_weights=True)
    assert rel_err(f64(bufs.o_latent), ref["o_lat"]) <= REL_TOL
    assert rel_err(f64(out)[:, 0], ref["out"]) <= REL_TOL
    check_rowsums(ref, f64(bufs.lse), None, bf16_query_scores(ref, w.q_pe, slot_rows(w), w.scale))
