"""GPU parity of mla_output_proj (the output projection after the value-up,
"Attention update" page, mla-output) against the fp64 oracle on sampled
batch rows: within 1e-2 * max|ref| (fp32 accumulation over 16384 products,
one rounding to bf16), across one and two 32-row batch tiles, a batch split
over two launches (64 + 36 rows), and strided input and output rows."""
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
