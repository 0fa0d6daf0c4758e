"""Checks that pin the prefill oracle (oracle.prefill, the full-sequence MHA
form of the "Queries" page's prefill excerpt) to facts other than itself.

Each ``pin_*`` takes a prefill callable with the signature of
``oracle.prefill`` and raises AssertionError when it disagrees with:

  * a library attention routine: with every causal key selected the result
    is causal attention, torch scaled_dot_product_attention(is_causal=True)
    in fp64 on the up-projected keys [W_UK c_t | k_pe_t] and values W_UV c_t;
  * the decode oracle (the absorbed gather form, itself pinned in
    tests/pins.py): query s of the prompt equals one decode query over the
    cache positions 0 .. s with the same index row (positions after s
    dropped by the causal mask);
  * causality: no query depends on a later key's latent or rotary key;
  * a closed form: the first query attends only key 0, so its output is
    W_UV c_0 exactly;
  * the index mask: an unselected key's latent changes nothing, and the
    attended set is the selection cut by the causal mask.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

SMALL = dict(H=4, Dn=8, Dc=16, Dr=4, Dv=8)
REAL = dict(H=128, Dn=128, Dc=512, Dr=64, Dv=128)


def make_prefill_inputs(seed, B, T, k, H, Dn, Dc, Dr, Dv, pad=0):
    """Random fp64 inputs.  Index rows of query s hold k distinct positions
    drawn from the whole prompt [0, T) (so that some lie after s and are
    removed by the causal mask) in random order, then ``pad`` -1s; k=None
    selects every key."""
    rng = np.random.default_rng(seed)
    q_nope = rng.standard_normal((B, T, H, Dn))
    q_pe = rng.standard_normal((B, T, H, Dr))
    kv = rng.standard_normal((B, T, Dc))
    pe = rng.standard_normal((B, T, Dr))
    wkv_b = rng.standard_normal((H * (Dn + Dv), Dc)) / np.sqrt(Dc)
    idx = None
    if k is not None:
        idx = np.full((B, T, min(k, T) + pad), -1, dtype=np.int64)
        for b in range(B):
            for s in range(T):
                r = rng.permutation(T)[: min(k, T)]
                if s not in r:            # every query selects itself, as a top-k would
                    r[0] = s
                idx[b, s, : len(r)] = r
    return dict(q_nope=q_nope, q_pe=q_pe, kv=kv, pe=pe, wkv_b=wkv_b, indices=idx,
                scale=(Dn + Dr) ** -0.5)


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _split_w(wkv_b, H, Dn, Dv):
    w = wkv_b.reshape(H, Dn + Dv, -1)
    return w[:, :Dn], w[:, Dn:]


def pin_prefill_sdpa_causal(pre):
    for dims in (SMALL, REAL):
        H, Dn, Dv = dims["H"], dims["Dn"], dims["Dv"]
        x = make_prefill_inputs(11, B=2, T=9, k=None, **dims)
        got = pre(**x)["out"]
        w_uk, w_uv = _split_w(x["wkv_b"], H, Dn, Dv)
        for b in range(2):
            kv = torch.from_numpy(x["kv"][b])                                   # [T, Dc]
            k_nope = torch.einsum("hdc,tc->htd", torch.from_numpy(w_uk), kv)   # [H, T, Dn]
            v = torch.einsum("hdc,tc->htd", torch.from_numpy(w_uv), kv)        # [H, T, Dv]
            k_pe = torch.from_numpy(x["pe"][b])[None].expand(H, -1, -1)
            k = torch.cat([k_nope, k_pe], -1)
            q = torch.cat([torch.from_numpy(x["q_nope"][b]), torch.from_numpy(x["q_pe"][b])], -1).transpose(0, 1)
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=x["scale"])
            assert _rel(got[b], ref.transpose(0, 1).numpy()) <= 1e-12


def pin_prefill_vs_decode(pre):
    for dims in (SMALL, REAL):
        x = make_prefill_inputs(12, B=2, T=7, k=4, pad=2, **dims)
        got = pre(**x)
        for b in range(2):
            for s in range(7):
                row = x["indices"][b, s].copy()
                row[row > s] = -1
                d = oracle.decode(x["q_nope"][b:b + 1, s], x["q_pe"][b:b + 1, s], x["kv"][b:b + 1],
                                  x["pe"][b:b + 1], x["wkv_b"], np.array([s + 1], dtype=np.int32),
                                  row[None], x["scale"])
                assert _rel(got["out"][b, s], d["out"][0]) <= 1e-12
                assert np.allclose(got["lse"][b, s], d["lse"][0], rtol=0, atol=1e-12)


def pin_prefill_causality(pre):
    x = make_prefill_inputs(13, B=1, T=8, k=5, **SMALL)
    base = pre(**x)["out"]
    s0 = 4
    y = dict(x)
    y["kv"] = x["kv"].copy()
    y["pe"] = x["pe"].copy()
    y["kv"][:, s0 + 1:] += 3.0
    y["pe"][:, s0 + 1:] -= 2.0
    moved = pre(**y)["out"]
    assert np.array_equal(moved[:, : s0 + 1], base[:, : s0 + 1])
    assert not np.allclose(moved[:, s0 + 1:], base[:, s0 + 1:])


def pin_prefill_first_token(pre):
    for dims in (SMALL, REAL):
        H, Dn, Dv = dims["H"], dims["Dn"], dims["Dv"]
        x = make_prefill_inputs(14, B=2, T=5, k=3, **dims)
        got = pre(**x)["out"]
        _, w_uv = _split_w(x["wkv_b"], H, Dn, Dv)
        for b in range(2):
            ref = np.einsum("hdc,c->hd", w_uv, x["kv"][b, 0])
            assert _rel(got[b, 0], ref) <= 1e-13


def pin_prefill_index_mask(pre):
    x = make_prefill_inputs(15, B=1, T=10, k=3, pad=1, **SMALL)
    res = pre(**x, want_attended=True)
    att = res["attended"][0]
    for s in range(10):
        row = x["indices"][0, s]
        want = sorted({int(t) for t in row if 0 <= t <= s})
        assert list(np.nonzero(att[s])[0]) == want
    # A key nobody attends: changing it changes nothing.
    free = [t for t in range(10) if not att[:, t].any()]
    if free:
        y = dict(x)
        y["kv"] = x["kv"].copy()
        y["kv"][0, free] += 5.0
        assert np.array_equal(pre(**y)["out"], res["out"])


PREFILL_PINS = [pin_prefill_sdpa_causal, pin_prefill_vs_decode, pin_prefill_causality,
                pin_prefill_first_token, pin_prefill_index_mask]
