"""Dense masked formulations of the decode step in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  These exist to pin the
C gather oracle; they are small-input checkers, not the timed oracle.

absorbed_dense()      F2: the decode branch as the "Query-key similarity" page
                      states it: absorb W_UK into the query, score every cached
                      position, add the -inf index mask, softmax over all
                      positions, mix the latents, project with W_UV ("Apply
                      value weights" page, formula O_i).
non_absorbed_dense()  F1: the full-sequence formulation of the "Queries" page
                      (prefill excerpt), specialised to one query position and
                      no causal mask: up-project every cached latent into
                      per-head k_nope and v, join k_nope with the shared rotary
                      key, score, mask, softmax, mix v.

"Apply value weights" page, Explanation: mixing latents first and projecting
after equals projecting every latent first, so F1 == F2 == the gather oracle in
exact arithmetic.  The tests check exactly that.
"""
from __future__ import annotations

import numpy as np


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis ("Softmax" page, formula for A)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def index_mask(indices_row, L: int) -> np.ndarray:
    """-inf everywhere, 0 scattered at the selected positions; -1 is padding."""
    mask = np.full(L, -np.inf)
    for t in np.asarray(indices_row).tolist():
        if t == -1:
            continue
        if not 0 <= t < L:
            raise IndexError(t)
        mask[t] = 0.0
    return mask


def absorbed_dense(q_nope, q_pe, kv, pe, wkv_b, seq_lens, indices, scale):
    """F2.  Arrays: q_nope [B,H,Dn], q_pe [B,H,Dr], kv [B,L,Dc], pe [B,L,Dr],
    wkv_b [H*(Dn+Dv), Dc], seq_lens [B], indices [B,k] or None.

    Returns (out [B,H,Dv], A list of [H, L_b] weights, q_abs [B,H,Dc]).
    """
    B, H, Dn = q_nope.shape
    Dc = kv.shape[2]
    w = wkv_b.reshape(H, -1, Dc)              # [H, Dn+Dv, Dc]
    w_uk = w[:, :Dn, :]                       # [H, Dn, Dc]
    w_uv = w[:, Dn:, :]                       # [H, Dv, Dc]
    q_abs = np.einsum("bhd,hdc->bhc", q_nope, w_uk)
    outs, weights = [], []
    for b in range(B):
        L = int(seq_lens[b])
        s = (q_abs[b] @ kv[b, :L].T + q_pe[b] @ pe[b, :L].T) * scale    # [H, L]
        if indices is not None:
            s = s + index_mask(indices[b], L)[None, :]
        a = _softmax_rows(s)
        x = a @ kv[b, :L]                                                # [H, Dc]
        outs.append(np.einsum("hc,hdc->hd", x, w_uv))
        weights.append(a)
    return np.stack(outs), weights, q_abs


def non_absorbed_dense(q_nope, q_pe, kv, pe, wkv_b, seq_lens, indices, scale):
    """F1.  Same arguments and outputs (without q_abs) as :func:`absorbed_dense`."""
    B, H, Dn = q_nope.shape
    Dc = kv.shape[2]
    per_head = wkv_b.shape[0] // H
    Dv = per_head - Dn
    outs, weights = [], []
    for b in range(B):
        L = int(seq_lens[b])
        # Linear(kv_lora_rank -> H*(Dn+Dv)) applied to every cached latent.
        up = (kv[b, :L] @ wkv_b.T).reshape(L, H, per_head)
        k_nope, v = up[:, :, :Dn], up[:, :, Dn:]                     # [L,H,Dn], [L,H,Dv]
        k = np.concatenate(
            [k_nope, np.broadcast_to(pe[b, :L, None, :], (L, H, pe.shape[2]))], axis=-1
        )                                                            # [L,H,Dn+Dr]
        q = np.concatenate([q_nope[b], q_pe[b]], axis=-1)            # [H,Dn+Dr]
        s = np.einsum("hd,thd->ht", q, k) * scale
        if indices is not None:
            s = s + index_mask(indices[b], L)[None, :]
        a = _softmax_rows(s)
        outs.append(np.einsum("ht,thd->hd", a, v))
        weights.append(a)
    assert outs[0].shape[-1] == Dv
    return np.stack(outs), weights
