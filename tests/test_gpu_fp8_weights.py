"""The block-scaled fp8 wkv_b read directly by absorb and value-up
(mla_absorb_q_fp8, mla_value_up_fp8, mla_combine_value_up_fp8, through the
C ABI): the bf16 weights the kernels form in registers equal the oracle's
dequantisation bit for bit (including products that fp32 rounds onto a bf16
tie, in blocks that take the exact rounding path and blocks that do not, and
every finite code; the two NaN codes give a NaN); the fp8 calls then give exactly the
outputs of the bf16 calls on the dequantised copy; and the dense fp8 workload
at full size matches the oracle ("Query-key similarity" page, code excerpt:
a quantised wkv_b dequantised through its block scales)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_amd import workload
from tests.gpu_common import REL_TOL, f64, gather_rows_for_oracle, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


def _formed(mla, codes, scales):
    """Weights as formed in registers: W_UK rows by the absorb, W_UV rows by
    the value-up (run on small dummy inputs)."""
    dev = "cuda"
    c, s = codes.to(dev), scales.to(dev)
    formed = torch.full((128 * 256, 512), -1, dtype=torch.int16, device=dev)
    q = torch.zeros((1, 1, 128, 128), dtype=torch.bfloat16, device=dev)
    mla.mla_absorb_q_fp8(q, c, s, w_formed=formed)
    o = torch.zeros((1, 128, 512), dtype=torch.bfloat16, device=dev)
    mla.mla_value_up_fp8(o, c, s, w_formed=formed)
    torch.cuda.synchronize()
    return formed.cpu().numpy().view(np.uint16)


def _tie_scales(seed=1):
    """One scale per 128 x 128 block, each chosen so that for one code v the
    fp32 product fl(v * s) has low 16 bits 0x8000 (a bf16 tie) while the
    exact product differs from it: rounding fl(v * s) to bf16 by
    round-to-nearest-even then gives the wrong neighbour half the time."""
    rng = np.random.default_rng(seed)
    vals = torch.arange(256, dtype=torch.int64).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    out = []
    while len(out) < 1024:
        v = float(vals[int(rng.integers(1, 127))])
        if v == 0 or np.frexp(v)[0] == 0.5:          # a power of two multiplies exactly
            continue
        p = np.float32(rng.uniform(v * 2.0 ** -8, v * 2.0 ** -4))
        pb = (p.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
        s = np.float32(np.float64(pb.view(np.float32)) / v)
        if not (2.0 ** -8 <= s <= 2.0 ** -4):
            continue
        if (np.float32(v) * s).view(np.uint32) != pb or np.float64(v) * np.float64(s) == np.float64(pb.view(np.float32)):
            continue
        out.append(float(s))
    return torch.tensor(out, dtype=torch.float32).view(256, 4)


def _ties(codes, scales):
    """Products whose fp32 value lies on a bf16 tie while the exact value does not."""
    v = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    sc = np.repeat(np.repeat(scales.numpy().astype(np.float64), 128, 0), 128, 1)
    p = (v * sc).astype(np.float32)
    return ((p.view(np.uint32) & 0xFFFF) == 0x8000) & (p.astype(np.float64) != v * sc)


def test_formed_weights_bit_exact(mla):
    codes, scales = workload.fp8_weights(128 * 256, 512, seed=5000)
    bits, _ = oracle.dequant_fp8(codes, scales)
    assert np.array_equal(_formed(mla, codes, scales), bits)


def test_formed_weights_all_codes_and_ties(mla):
    """Every code in every scale block; the even blocks' scales put fp32
    products on bf16 ties (the kernels take their exact rounding path there),
    the odd blocks' are drawn across [2^-8, 2^-4]."""
    rows, cols = 128 * 256, 512
    codes = (torch.arange(rows * cols, dtype=torch.int64) * 7 % 256).to(torch.uint8).view(rows, cols)
    g = torch.Generator().manual_seed(5)
    scales = torch.exp2(torch.empty((256, 4)).uniform_(-8.0, -4.0, generator=g)).float()
    tie = _tie_scales()
    scales.view(-1)[0::2] = tie.view(-1)[0::2]
    ties = _ties(codes, scales)
    assert int(ties.sum()) > 1000
    bits, _ = oracle.dequant_fp8(codes, scales)
    # Rounding the fp32 product directly would miss some of them.
    v = codes.view(torch.float8_e4m3fn).float()
    naive = (v * torch.from_numpy(np.repeat(np.repeat(scales.numpy(), 128, 0), 128, 1))).to(torch.bfloat16)
    assert not np.array_equal(naive.view(torch.int16).numpy().view(np.uint16)[ties], bits[ties])
    got = _formed(mla, codes, scales)
    nan_code = (codes.numpy() & 0x7F) == 0x7F
    assert np.array_equal(got[~nan_code], bits[~nan_code])
    assert np.all(((got[nan_code] & 0x7F80) == 0x7F80) & ((got[nan_code] & 0x7F) != 0))


def test_fp8_calls_equal_bf16_calls(mla):
    dev = "cuda"
    codes, scales = workload.fp8_weights(128 * 256, 512, seed=5100)
    c, s = codes.to(dev), scales.to(dev)
    wbf = mla.mla_dequant_wkv_b_fp8(c, s)
    g = torch.Generator().manual_seed(9)
    B = 45
    q = torch.randn((B, 1, 128, 128), generator=g).to(torch.bfloat16).to(dev)
    assert torch.equal(mla.mla_absorb_q_fp8(q, c, s), mla.mla_absorb_q(q, wbf))
    # 300 rows: ten 32-row query tiles in three groups, the later ones
    # staged while the one before is computed, in both tile sets.
    q3 = torch.randn((300, 1, 128, 128), generator=g).to(torch.bfloat16).to(dev)
    assert torch.equal(mla.mla_absorb_q_fp8(q3, c, s), mla.mla_absorb_q(q3, wbf))
    o = torch.randn((B, 128, 512), generator=g).to(torch.bfloat16).to(dev)
    assert torch.equal(mla.mla_value_up_fp8(o, c, s), mla.mla_value_up(o, wbf))
    for S in (2, 4):
        w = workload.make("sparse_b32_l4096_k2048", B=B, L=600, k=300)
        gw = {k: getattr(w, k).to(dev) for k in ("q_pe", "cache", "seq_lens", "indices")}
        bufs = mla.DecodeBuffers.allocate(B, w.k_max, False, num_splits=S)
        qa = mla.mla_absorb_q(q, wbf)
        mla.mla_sparse_decode(qa, gw["q_pe"], gw["cache"][..., :512], gw["cache"][..., 512:], gw["seq_lens"],
                              w.max_len, gw["indices"], w.scale, S, bufs.workspace, bufs.o_latent, bufs.lse)
        lse1, lse2 = torch.empty_like(bufs.lse), torch.empty_like(bufs.lse)
        out1 = mla.mla_combine_value_up(bufs.workspace, B, S, wbf, lse=lse1)
        out2 = mla.mla_combine_value_up_fp8(bufs.workspace, B, S, c, s, lse=lse2)
        torch.cuda.synchronize()
        assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_fp8_workload_full_size(mla):
    """The dense fp8 workload (B = 64, 8192 positions) with the fp8 weight
    read directly by absorb and value-up, against the oracle on sampled
    sequences and bit for bit against the path through the bf16 copy."""
    name = "dense_fp8w_b64_l8192"
    print(f"[fp8] {name}", flush=True)
    dev = "cuda"
    w = workload.make(name, device="cpu", cache_device=dev)
    c, s = w.wkv_b_fp8.to(dev), w.wkv_b_scale.to(dev)
    q_nope, q_pe, lens = w.q_nope.to(dev), w.q_pe.to(dev), w.seq_lens.to(dev)
    S = mla.mla_plan(w.B, w.k_max, True)
    bufs = mla.DecodeBuffers.allocate(w.B, w.k_max, True, num_splits=S)
    qa = mla.mla_absorb_q_fp8(q_nope, c, s)
    mla.mla_sparse_decode(qa, q_pe, w.kv, w.pe, lens, w.max_len, None, w.scale, S, bufs.workspace, bufs.o_latent,
                          bufs.lse, k_max=w.k_max)
    out = mla.mla_combine_value_up_fp8(bufs.workspace, w.B, S, c, s, lse=bufs.lse).clone()
    wbf = mla.mla_dequant_wkv_b_fp8(c, s)
    ref_path = mla.decode_step(bufs, q_nope, q_pe, w.kv, w.pe, wbf, lens, w.max_len, None, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_path)
    rows = [0, 31, 63]
    w.seq_lens, w.indices = lens, None
    kv, pe, klens, kidx = gather_rows_for_oracle(w, rows)
    bits, _ = oracle.dequant_fp8(w.wkv_b_fp8, w.wkv_b_scale)
    wref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    sel = torch.tensor(rows)
    ref = oracle.decode(w.q_nope[sel], w.q_pe[sel], kv, pe, wref, klens, kidx, w.scale)
    assert rel_err(f64(out)[rows, 0], ref["out"]) <= REL_TOL
