"""GPU parity of mla_output_proj (the output projection after the value-up,
"Attention update" page, mla-output) against the fp64 oracle on sampled
batch rows: within 1e-2 * max|ref| (fp32 accumulation over 16384 products,
one rounding to bf16), across one and two 32-row batch tiles, a batch split
over two launches (64 + 36 rows), and strided input and output rows.  The
repacked weight (mla_output_proj_pack) is checked element for element against
its definition, and mla_output_proj_packed bit for bit against
mla_output_proj on the unpacked weight.  mla_output_proj_split (the inputs
split in four, fp32 partial sums added by a second launch) is checked
against the oracle on the same rows, and on every row against
mla_output_proj within two bf16 steps of the largest output (the two sum in
different orders)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_amd import workload
from tests.gpu_common import REL_TOL, f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mla_amd import binding
    return binding


@pytest.fixture(scope="module")
def inputs():
    x, wo = workload.output_proj_inputs(100)
    return x, wo, x.cuda(), wo.cuda()


@pytest.mark.parametrize("B,rows", [(1, [0]), (37, [0, 31, 32, 36]), (64, [5, 63]), (100, [0, 63, 64, 99])])
def test_output_proj(mla, inputs, B, rows):
    x, wo, xg, wog = inputs
    out = mla.mla_output_proj(xg[:B], wog)
    torch.cuda.synchronize()
    ref = oracle.output_proj(x[rows], wo)
    assert rel_err(f64(out)[rows, 0], ref) <= REL_TOL


def test_output_proj_strided_rows(mla, inputs):
    x, wo, xg, wog = inputs
    B = 40
    xs = torch.zeros((B, 16384 + 64), dtype=torch.bfloat16, device="cuda")
    xs[:, :16384] = xg[:B].reshape(B, -1)
    big = torch.full((B, 7200), 7.0, dtype=torch.bfloat16, device="cuda")
    mla.mla_output_proj(xs[:, :16384], wog, out=big[:, :7168])
    torch.cuda.synchronize()
    rows = [0, 39]
    ref = oracle.output_proj(x[rows], wo)
    assert rel_err(f64(big)[rows, :7168], ref) <= REL_TOL
    assert torch.all(big[:, 7168:] == 7.0)  # nothing written past each row's 7168 values


def test_output_proj_pack_layout(mla, inputs):
    _, _, _, wog = inputs
    packed = mla.mla_output_proj_pack(wog)
    torch.cuda.synchronize()
    # packed[g][c][r][k] = wo[28 g + r][256 c + k]
    ref = wog.view(256, 28, 64, 256).permute(0, 2, 1, 3).contiguous().view(7168, 16384)
    assert torch.equal(packed.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("B", [1, 9, 32, 33, 64, 100])
def test_output_proj_packed_bit_identical(mla, inputs, B):
    x, wo, xg, wog = inputs
    packed = mla.mla_output_proj_pack(wog)
    a = mla.mla_output_proj(xg[:B], wog)
    b = mla.mla_output_proj_packed(xg[:B], packed)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.output_proj(x[[0, B - 1]], wo)
    assert rel_err(f64(b)[[0, B - 1], 0], ref) <= REL_TOL


@pytest.mark.parametrize("B,rows", [(1, [0]), (32, [0, 31]), (37, [0, 31, 32, 36]), (64, [5, 63]),
                                    (100, [0, 63, 64, 99])])
def test_output_proj_split(mla, inputs, B, rows):
    x, wo, xg, wog = inputs
    ws = torch.full((mla.mla_output_proj_split_workspace_bytes(B),), 0xFF, dtype=torch.uint8, device="cuda")
    out = mla.mla_output_proj_split(xg[:B], wog, ws)
    plain = mla.mla_output_proj(xg[:B], wog)
    torch.cuda.synchronize()
    ref = oracle.output_proj(x[rows], wo)
    assert rel_err(f64(out)[rows, 0], ref) <= REL_TOL
    assert rel_err(f64(out), f64(plain)) <= 2 * 2.0 ** -8


def test_output_proj_split_strided_and_errors(mla, inputs):
    x, wo, xg, wog = inputs
    B = 40
    xs = torch.zeros((B, 16384 + 64), dtype=torch.bfloat16, device="cuda")
    xs[:, :16384] = xg[:B].reshape(B, -1)
    big = torch.full((B, 7200), 7.0, dtype=torch.bfloat16, device="cuda")
    mla.mla_output_proj_split(xs[:, :16384], wog, out=big[:, :7168])
    torch.cuda.synchronize()
    rows = [0, 39]
    ref = oracle.output_proj(x[rows], wo)
    assert rel_err(f64(big)[rows, :7168], ref) <= REL_TOL
    assert torch.all(big[:, 7168:] == 7.0)
    small = torch.empty(mla.mla_output_proj_split_workspace_bytes(B) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mla.MLAError):
        mla.mla_output_proj_split(xg[:B], wog, small)
