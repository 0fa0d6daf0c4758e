"""CPU tests: the fp64 oracle against what the pages and the mathematics fix."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.decode)


def test_out_of_range_index_raises():
    x = pins.make_inputs(20, 1, 6, 2, **pins.SMALL)
    x["indices"][0, 0] = 6
    with pytest.raises(IndexError):
        oracle.decode(**x)
    x["indices"][0, 0] = -2
    with pytest.raises(IndexError):
        oracle.decode(**x)


def test_empty_selection_is_nan():
    """All -inf scores: softmax is 0/0 (NaN); the status flags it."""
    x = pins.make_inputs(21, 2, 6, 2, **pins.SMALL)
    x["indices"][1, :] = -1
    got = oracle.decode(**x)
    assert got["status"] & oracle.ORACLE_ERR_EMPTY
    assert np.all(np.isnan(got["out"][1])) and np.all(np.isfinite(got["out"][0]))
    assert np.all(got["lse"][1] == -np.inf)


def test_fp8_e4m3_decode_matches_torch():
    """All 256 E4M3FN codes against torch's float8_e4m3fn conversion."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.e4m3_to_double(0x7E) == 448.0 and oracle.e4m3_to_double(0x01) == 2.0 ** -9


def _bf16_exact_rne(x: float) -> int:
    """Reference rounding with exact rationals: nearest bf16, ties to even."""
    if x == 0:
        return 0x8000 if math.copysign(1, x) < 0 else 0
    fx = Fraction(x)
    sign = 0x8000 if fx < 0 else 0
    ax = abs(fx)
    e = math.floor(math.log2(ax))
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 7)
    q = ax / ulp
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(n * ulp)
    bits = np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16
    return int(bits) | sign


def test_bf16_rounding():
    """The oracle's double -> bf16 rounding: against torch's fp32 -> bf16 on
    fp32-representable values, and against exact rational rounding on ties
    and near-ties that a float intermediate would round twice."""
    rng = np.random.default_rng(3)
    vals = (rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000))).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([oracle.double_to_bf16_bits(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    cases = []
    for base in (1.0, 1.0078125, 3.5, -0.0390625, 2.0 ** -100):
        ulp = abs(base) * 2.0 ** -7
        for frac in (0.5, 0.5 + 2.0 ** -30, 0.5 - 2.0 ** -30, 1.5, 0.25):
            cases.append(base + math.copysign(ulp * frac, base))
    for v in cases:
        assert oracle.double_to_bf16_bits(v) == _bf16_exact_rne(v), v


def test_dequant_fp8_exact():
    """Dequantisation: exact product (checked with rationals) then one RNE."""
    rng = np.random.default_rng(4)
    rows, cols = 256, 256
    codes = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C     # no NaN codes in weights
    scales = np.exp2(rng.uniform(-8, -4, (2, 2))).astype(np.float32)
    bits, exact = oracle.dequant_fp8(codes, scales)
    sample = rng.integers(0, rows * cols, 400)
    for flat in sample.tolist():
        i, j = divmod(flat, cols)
        v = Fraction(oracle.e4m3_to_double(int(codes[i, j]))) * Fraction(float(scales[i // 128, j // 128]))
        assert Fraction(exact[i, j]) == v
        assert bits[i, j] == _bf16_exact_rne(float(v)) or v == 0


def test_step_absorb_identity_and_agreement():
    """oracle.absorb: W_UK = [I | 0] gives [q_nope, 0] exactly, and it equals
    the absorbed query the full oracle reports."""
    x = pins.make_inputs(30, 2, 6, 3, **pins.REAL)
    full = oracle.decode(**x)
    assert np.array_equal(oracle.absorb(x["q_nope"], x["wkv_b"]), full["q_abs"])
    H, Dn, Dc, Dv = 128, 128, 512, 128
    w = x["wkv_b"].reshape(H, Dn + Dv, Dc).copy()
    w[:, :Dn, :] = 0.0
    w[:, np.arange(Dn), np.arange(Dn)] = 1.0
    got = oracle.absorb(x["q_nope"], w.reshape(-1, Dc))
    assert np.array_equal(got[:, :, :Dn], x["q_nope"]) and np.all(got[:, :, Dn:] == 0.0)


def test_step_value_up_identity_and_agreement():
    """oracle.value_up: W_UV = [I | 0] gives the first 128 latent features
    exactly, and it equals the output the full oracle reports."""
    x = pins.make_inputs(31, 2, 6, 3, **pins.REAL)
    full = oracle.decode(**x)
    assert np.array_equal(oracle.value_up(full["o_lat"], x["wkv_b"]), full["out"])
    H, Dn, Dc, Dv = 128, 128, 512, 128
    w = x["wkv_b"].reshape(H, Dn + Dv, Dc).copy()
    w[:, Dn:, :] = 0.0
    w[:, Dn + np.arange(Dv), np.arange(Dv)] = 1.0
    o = np.random.default_rng(1).standard_normal((2, H, Dc))
    assert np.array_equal(oracle.value_up(o, w.reshape(-1, Dc)), o[:, :, :Dv])


def _exact_output_proj(x, wo):
    """Brute force with exact rational arithmetic (Python fractions): each
    sum of products written out, then rounded once to float."""
    from fractions import Fraction
    B, Din = x.shape
    Dout = wo.shape[0]
    out = np.empty((B, Dout))
    for b in range(B):
        for o in range(Dout):
            out[b, o] = float(sum(Fraction(float(x[b, i])) * Fraction(float(wo[o, i])) for i in range(Din)))
    return out


def test_output_proj_brute_force():
    # "Attention update" page, mla-output: out[b][o] = sum_i x[b][i] wo[o][i]
    # on non-square shapes (a transposed operand or a dropped term fails).
    g = torch.Generator().manual_seed(607)
    for B, Din, Dout in [(2, 6, 3), (3, 5, 7), (1, 16, 2)]:
        x = torch.randn(B, Din, generator=g).to(torch.bfloat16)
        wo = torch.randn(Dout, Din, generator=g).to(torch.bfloat16)
        got = oracle.output_proj(x, wo)
        ref = _exact_output_proj(x.double().numpy(), wo.double().numpy())
        assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


def test_output_proj_selection_at_the_real_shape():
    # One 1 per row of wo: out[b][o] = x[b][perm(o)] exactly, with x the
    # flattened [B, 1, 128, 128] head outputs and the model width 7168.
    g = torch.Generator().manual_seed(608)
    x = torch.randn(2, 1, 128, 128, generator=g).to(torch.bfloat16)
    perm = torch.randperm(128 * 128, generator=g)[:7168]
    wo = torch.zeros(7168, 128 * 128, dtype=torch.bfloat16)
    wo[torch.arange(7168), perm] = 1
    got = oracle.output_proj(x, wo)
    assert np.array_equal(got, x.reshape(2, -1).double().numpy()[:, perm.numpy()])


# Prefill oracle (full-sequence MHA form), pinned by tests/pins_prefill.py.
from tests import pins_prefill  # noqa: E402


@pytest.mark.parametrize("pin", pins_prefill.PREFILL_PINS, ids=lambda p: p.__name__)
def test_prefill_pin(pin):
    pin(oracle.prefill)
