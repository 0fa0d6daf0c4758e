"""GPU parity of the value-up at large batches of merged rows (mla_value_up
with 512 rows or more: workgroups that form W_UV,h once and stream the
batch's 32-row tiles, as the prefill's B * T rows use it).  Its products
are those of the per-tile kernel that smaller calls use, in the same order,
so the results are compared bit for bit with the same rows passed in
64-row calls; sampled rows also against the oracle's value-up ("Apply value
weights" page, formula O_i), within 4e-3 of max|ref| (one bf16 rounding of
an fp32 sum of 512 products)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_amd import workload
from tests.gpu_common import f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


def _in_slices(fn, o, rows=64):
    return torch.cat([fn(o[i:i + rows]) for i in range(0, o.shape[0], rows)], 0)


@pytest.mark.parametrize("B,H", [(4096, 128), (600, 128), (1000, 16), (512, 64)])
def test_streamed_value_up_equals_tiled(mla, B, H):
    gen = torch.Generator().manual_seed(B + H)
    o = torch.randn((B, H, 512), generator=gen).to(torch.bfloat16)
    w = workload.make("sparse_b32_l4096_k2048", B=1, L=8, k=4).wkv_b[: H * 256].contiguous()
    og, wg = o.cuda(), w.cuda()
    full = mla.mla_value_up(og, wg)
    tiled = _in_slices(lambda x: mla.mla_value_up(x.contiguous(), wg), og)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), tiled.view(torch.int16))
    rows = [0, B // 2, B - 1]
    ref = oracle.value_up(o[rows], w) if H == 128 else None
    if ref is not None:
        assert rel_err(f64(full)[rows, 0], ref) <= 4e-3


def test_streamed_value_up_fp8(mla):
    """fp8 weights read directly at 800 rows: bit-identical to the bf16 call
    on the one-time dequantised copy, and the weights formed in registers
    equal the oracle's dequantisation on the W_UV rows."""
    B = 800
    w = workload.make("dense_fp8w_b64_l8192", B=1, L=8)
    codes, scales = w.wkv_b_fp8, w.wkv_b_scale
    o = torch.randn((B, 128, 512), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    cg, sg = codes.cuda(), scales.cuda()
    bf = mla.mla_dequant_wkv_b_fp8(cg, sg)
    formed = torch.zeros((32768, 512), dtype=torch.bfloat16, device="cuda")
    a = mla.mla_value_up_fp8(o, cg, sg, w_formed=formed)
    b = mla.mla_value_up(o, bf)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    bits, _ = oracle.dequant_fp8(codes, scales)
    got = formed.view(torch.int16).cpu().numpy().view(np.uint16).reshape(128, 256, 512)[:, 128:]
    exp = bits.reshape(128, 256, 512)[:, 128:]
    both_nan = ((got & 0x7FFF) > 0x7F80) & ((exp & 0x7FFF) > 0x7F80)
    assert np.array_equal(np.where(both_nan, 0, got), np.where(both_nan, 0, exp))
