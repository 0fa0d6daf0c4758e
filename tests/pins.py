"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function takes a decode callable with the signature of
``oracle.decode`` and raises AssertionError when the callable disagrees with:

  * the non-absorbed formulation ("Queries" page, prefill excerpt) -- the
    absorption identity of the "Apply value weights" page, Explanation;
  * the dense masked absorbed formulation (decode excerpt on the
    "Query-key similarity" page) -- gather == dense mask;
  * the softmax definition ("Softmax" page, formula for A): rows sum to one,
    exactly zero weight off the selected set;
  * a library attention routine (torch scaled_dot_product_attention in fp64)
    when every position is selected;
  * closed forms: one selected position gives W_UV c_j; a zero query gives the
    mean of the selected latents; W_UK = [I | 0] gives q~ = [q_nope, 0];
  * invariances of the set-valued mask (order, repeats);
  * exact 50-digit decimal arithmetic on tiny inputs.

tests/test_oracle_pins.py runs them against the oracle; tests/test_oracle_mutants.py
runs them against deliberately broken builds of the oracle and expects failures.
"""
from __future__ import annotations

from decimal import Decimal, getcontext

import numpy as np
import torch

from oracle.formulations import absorbed_dense, non_absorbed_dense

SMALL = dict(H=4, Dn=8, Dc=16, Dr=4, Dv=8)
REAL = dict(H=128, Dn=128, Dc=512, Dr=64, Dv=128)


def make_inputs(seed, B, L, k, H, Dn, Dc, Dr, Dv, lens=None, pad=0, dup=0):
    """Random fp64 inputs.  Index rows hold min(k, L_b) distinct positions in
    random order, then ``dup`` repeats of earlier entries, then ``pad`` -1s."""
    rng = np.random.default_rng(seed)
    q_nope = rng.standard_normal((B, H, Dn))
    q_pe = rng.standard_normal((B, H, Dr))
    kv = rng.standard_normal((B, L, Dc))
    pe = rng.standard_normal((B, L, Dr))
    wkv_b = rng.standard_normal((H * (Dn + Dv), Dc)) / np.sqrt(Dc)
    lens = np.full(B, L, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
    idx = None
    if k is not None:
        rows = []
        for b in range(B):
            r = list(rng.permutation(int(lens[b]))[: min(k, int(lens[b]))])
            r += [r[i % len(r)] for i in range(dup)] if r else []
            r += [-1] * pad
            rows.append(r)
        width = max(len(r) for r in rows)
        idx = np.array([r + [-1] * (width - len(r)) for r in rows], dtype=np.int64)
    scale = (Dn + Dr) ** -0.5
    return dict(q_nope=q_nope, q_pe=q_pe, kv=kv, pe=pe, wkv_b=wkv_b,
                seq_lens=lens, indices=idx, scale=scale)


def _rel(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def pin_absorption_identity(dec):
    """F1 (non-absorbed) == oracle, small and real dims, ragged, padded."""
    for seed, dims, B, L, k, lens in [
        (1, SMALL, 3, 12, 5, [12, 7, 9]),
        (2, SMALL, 2, 9, 9, None),
        (3, REAL, 2, 24, 9, [24, 13]),
    ]:
        x = make_inputs(seed, B, L, k, **dims, lens=lens, pad=2)
        ref, _ = non_absorbed_dense(**x)
        got = dec(**x)["out"]
        r = _rel(got, ref)
        assert r <= 1e-12, f"absorption identity: rel err {r:.3e} (seed {seed})"


def pin_dense_vs_gather(dec):
    """F2 (dense -inf mask) == oracle, with repeats and -1 padding; q~ too."""
    x = make_inputs(4, 3, 15, 6, **SMALL, lens=[15, 4, 10], pad=3, dup=2)
    ref, _, qa = absorbed_dense(**x)
    got = dec(**x)
    assert _rel(got["out"], ref) <= 1e-12, "dense vs gather: out"
    assert _rel(got["q_abs"], qa) <= 1e-13, "dense vs gather: absorbed query"


def pin_softmax_rows(dec):
    """Weights of the distinct selected slots sum to 1; padding slots and
    unselected positions carry exactly zero weight; the attended set is the
    set of distinct valid indices."""
    x = make_inputs(5, 2, 20, 7, **SMALL, lens=[20, 11], pad=3)
    got = dec(**x, want_weights=True, want_attended=True)
    w = got["weights"]
    idx = x["indices"]
    for b in range(idx.shape[0]):
        valid = idx[b] >= 0
        s = w[b][:, valid].sum(axis=1)
        assert np.all(np.abs(s - 1.0) <= 1e-12), f"row sums {s}"
        assert np.all(w[b][:, ~valid] == 0.0), "padding slot has weight"
        expect = np.zeros(got["attended"].shape[1], dtype=np.uint8)
        expect[idx[b][valid]] = 1
        assert np.array_equal(got["attended"][b], expect), "attended set"
        # the dense formulation puts exactly zero weight off the set
    _, A, _ = absorbed_dense(**x)
    for b in range(idx.shape[0]):
        off = np.ones(A[b].shape[1], dtype=bool)
        off[idx[b][idx[b] >= 0]] = False
        assert np.all(A[b][:, off] == 0.0)


def pin_sdpa_all_selected(dec):
    """Selecting every position is ordinary MQA-style attention over the
    up-projected keys [W_UK c_t | k_pe_t] and values W_UV c_t: compare with
    torch's scaled_dot_product_attention in float64."""
    for seed, dims, B, L in [(6, SMALL, 2, 10), (7, REAL, 1, 33)]:
        x = make_inputs(seed, B, L, None, **dims)
        H, Dn, Dc = dims["H"], dims["Dn"], dims["Dc"]
        w = torch.from_numpy(x["wkv_b"]).view(H, -1, Dc)
        w_uk, w_uv = w[:, :Dn], w[:, Dn:]
        outs = []
        for b in range(B):
            c = torch.from_numpy(x["kv"][b])                      # [L, Dc]
            kr = torch.from_numpy(x["pe"][b])                     # [L, Dr]
            k_nope = torch.matmul(w_uk, c.T).transpose(1, 2)      # [H, L, Dn]
            k = torch.cat([k_nope, kr.expand(H, -1, -1)], dim=-1)  # [H, L, Dn+Dr]
            v = torch.matmul(w_uv, c.T).transpose(1, 2)           # [H, L, Dv]
            q = torch.cat([torch.from_numpy(x["q_nope"][b]),
                           torch.from_numpy(x["q_pe"][b])], dim=-1)[:, None, :]
            o = torch.nn.functional.scaled_dot_product_attention(
                q[None], k[None].contiguous(), v[None].contiguous(), scale=x["scale"])
            outs.append(o[0, :, 0, :].numpy())
        got = dec(**x)["out"]
        r = _rel(got, np.stack(outs))
        assert r <= 1e-12, f"sdpa: rel err {r:.3e}"


def pin_single_position(dec):
    """One selected position j: weight 1, so O_h = W_UV,h c_j (closed form)."""
    x = make_inputs(8, 2, 9, 1, **REAL, pad=2)
    got = dec(**x)
    H, Dn, Dc = REAL["H"], REAL["Dn"], REAL["Dc"]
    w_uv = x["wkv_b"].reshape(H, -1, Dc)[:, Dn:]
    for b in range(2):
        j = int(x["indices"][b][0])
        ref = w_uv @ x["kv"][b, j]                                # [H, Dv]
        assert _rel(got["out"][b], ref) <= 1e-13, "single position"
        assert np.array_equal(got["o_lat"][b], np.broadcast_to(x["kv"][b, j], (H, Dc)))


def pin_zero_query(dec):
    """q_nope = q_pe = 0: every selected position scores 0, the weights are
    uniform and O~ is the mean of the selected latents."""
    x = make_inputs(9, 2, 14, 5, **SMALL, lens=[14, 6], pad=1)
    x["q_nope"][:] = 0.0
    x["q_pe"][:] = 0.0
    got = dec(**x)
    for b in range(2):
        sel = x["indices"][b][x["indices"][b] >= 0]
        mean = x["kv"][b, sel].mean(axis=0)
        assert _rel(got["o_lat"][b], np.broadcast_to(mean, got["o_lat"][b].shape)) <= 1e-14
        assert np.allclose(got["lse"][b], np.log(len(sel)), rtol=0, atol=1e-14)


def pin_invariances(dec):
    """Permuting an index row or repeating entries leaves every output unchanged."""
    x = make_inputs(10, 2, 16, 6, **SMALL)
    base = dec(**x)
    rng = np.random.default_rng(0)
    perm = dict(x)
    perm["indices"] = np.stack([rng.permutation(r) for r in x["indices"]])
    rep = dict(x)
    rep["indices"] = np.concatenate([x["indices"], x["indices"][:, :3]], axis=1)
    for y in (perm, rep):
        got = dec(**y)
        for key in ("out", "lse", "o_lat"):
            assert np.array_equal(got[key], base[key]), key


def pin_identity_wuk(dec):
    """W_UK,h = [I | 0]: the absorbed query is [q_nope, 0, ..., 0] exactly."""
    x = make_inputs(11, 1, 5, 3, **REAL)
    H, Dn, Dc, Dv = REAL["H"], REAL["Dn"], REAL["Dc"], REAL["Dv"]
    w = x["wkv_b"].reshape(H, Dn + Dv, Dc)
    w[:, :Dn, :] = 0.0
    w[:, np.arange(Dn), np.arange(Dn)] = 1.0
    x["wkv_b"] = w.reshape(-1, Dc)
    got = dec(**x)
    expect = np.zeros((1, H, Dc))
    expect[:, :, :Dn] = x["q_nope"]
    assert np.array_equal(got["q_abs"], expect), "identity W_UK"


def _exact_decode(x):
    """Every step in 50-digit decimal arithmetic (tiny inputs only)."""
    getcontext().prec = 50
    D = Decimal
    B, H, Dn = x["q_nope"].shape
    Dc = x["kv"].shape[2]
    Dr = x["pe"].shape[2]
    Dv = x["wkv_b"].shape[0] // H - Dn
    W = [[D(float(v)) for v in row] for row in x["wkv_b"]]
    sc = D(float(x["scale"]))
    out = np.zeros((B, H, Dv))
    lse = np.zeros((B, H))
    for b in range(B):
        sel = sorted({int(t) for t in x["indices"][b] if t >= 0})
        for h in range(H):
            base = h * (Dn + Dv)
            qa = [sum(D(float(x["q_nope"][b, h, d])) * W[base + d][c] for d in range(Dn))
                  for c in range(Dc)]
            s = []
            for t in sel:
                lat = sum(qa[c] * D(float(x["kv"][b, t, c])) for c in range(Dc))
                rot = sum(D(float(x["q_pe"][b, h, r])) * D(float(x["pe"][b, t, r]))
                          for r in range(Dr))
                s.append((lat + rot) * sc)
            m = max(s)
            e = [(v - m).exp() for v in s]
            den = sum(e)
            a = [v / den for v in e]
            mix = [sum(a[j] * D(float(x["kv"][b, t, c])) for j, t in enumerate(sel))
                   for c in range(Dc)]
            for d in range(Dv):
                out[b, h, d] = float(sum(mix[c] * W[base + Dn + d][c] for c in range(Dc)))
            lse[b, h] = float(m + den.ln())
    return out, lse


def pin_brute_force(dec):
    """The oracle agrees with exact decimal arithmetic to fp64 rounding."""
    x = make_inputs(12, 2, 8, 4, H=2, Dn=3, Dc=5, Dr=2, Dv=3, lens=[8, 6], pad=1, dup=1)
    out, lse = _exact_decode(x)
    got = dec(**x)
    assert _rel(got["out"], out) <= 1e-13, "brute force out"
    assert _rel(got["lse"], lse) <= 1e-14, "brute force lse"


ALL_PINS = [
    pin_absorption_identity,
    pin_dense_vs_gather,
    pin_softmax_rows,
    pin_sdpa_all_selected,
    pin_single_position,
    pin_zero_query,
    pin_invariances,
    pin_identity_wuk,
    pin_brute_force,
]
