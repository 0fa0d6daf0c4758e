"""The rescale inputs (tests/rescale_inputs.py) against the oracle, on the CPU.

1. The oracle's exact scores show that the inputs make the lazy rule move the
   reference maximum of live accumulators, for even and odd heads, in splits
   of every size the GPU test runs, with a margin that no rounding of the
   kernel's fp32 scores can close.
2. The inputs are sensitive to the mistakes a rescale can make: a model of
   the split online softmax ("Softmax" page, formula for A, computed over
   blocks with the reference maximum moved lazily) run in fp64 on the
   oracle's scores reproduces the oracle's latent mix, and each planted
   mistake (no factor, the factor on the sum only, natural instead of base-2
   units, the factor applied after the block instead of before it) moves the
   result by more than the GPU bar of 1e-2 * max |O~_ref|.
"""
import numpy as np
import pytest
import torch

from sparse_mla_amd import workload
from tests.gpu_common import REL_TOL, oracle_ref, rel_err
from tests.rescale_inputs import BLK, LOG2E, THRESH, rescale_events, spike_workload, split_chunk

CONFIGS = [("sparse", 1), ("sparse", 2), ("sparse", 4), ("dense", 1), ("dense", 4)]


def _ref(mode, S):
    w = spike_workload(mode, S)
    return w, oracle_ref(w, want_weights=True)


@pytest.mark.parametrize("mode,S", CONFIGS)
def test_rescale_fires(mode, S):
    w, ref = _ref(mode, S)
    events, _ = rescale_events(ref["scores"], S, margin=0.5)
    assert events, "no rescale with a margin"
    heads = {h % 2 for (_, h, _, _) in events}
    assert heads == {0, 1}, "both head parities rescale"
    # Every split that holds at least three blocks rescales some head.
    chunk = split_chunk(w.k_max, S)
    for s in range(S):
        n = min(chunk, w.k_max - s * chunk)
        if n >= 3 * BLK:
            assert any(e[2] == s for e in events), f"split {s} never rescales"
    # Two rescales in one split for some head (level 1, then level 2).
    per = {}
    for (b, h, s, j) in events:
        per.setdefault((b, h, s), []).append(j)
    assert max(len(v) for v in per.values()) >= 2
    if mode == "sparse":
        # The split whose first block is fully masked still rescales later.
        b, s = (0, 1) if S > 1 else (1, 0)
        assert np.all(np.isneginf(ref["scores"][b, :, s * chunk: s * chunk + BLK]))
        assert any(e[0] == b and e[2] == s for e in events)


def _lazy_mix(scores, lat, S, mistake=None):
    """Split online softmax over 32-key blocks with the lazy reference
    maximum, then the log-sum-exp merge of the splits; fp64.  scores
    [H, k] (natural units, -inf masked), lat [k, 512] (rows of the slots)."""
    with np.errstate(invalid="ignore"):  # -inf - -inf where a head has no key yet
        return _lazy_mix_impl(scores, lat, S, mistake)


def _lazy_mix_impl(scores, lat, S, mistake):
    H, k = scores.shape
    chunk = split_chunk(k, S)
    u = scores * LOG2E
    parts = []
    for s in range(S):
        s0, s1 = s * chunk, min(k, (s + 1) * chunk)
        m_ref = np.full(H, -np.inf)
        l = np.zeros(H)
        acc = np.zeros((H, lat.shape[1]))
        for j0 in range(s0, s1, BLK):
            ub = u[:, j0:min(s1, j0 + BLK)]
            mb = ub.max(-1)
            need = mb > m_ref + THRESH
            resc = need & np.isfinite(m_ref)
            mnew = np.where(need, mb, m_ref)
            if mistake == "natural_units":
                alpha = np.where(resc, np.exp(m_ref - mnew), 1.0)
            else:
                alpha = np.where(resc, np.exp2(np.where(resc, m_ref - mnew, 0.0)), 1.0)
            ref_pt = np.where(np.isfinite(mnew), mnew, 0.0)
            p = np.exp2(ub - ref_pt[:, None])
            if mistake == "no_factor":
                pass
            elif mistake == "sum_only":
                l = l * alpha
            elif mistake == "after_block":
                l = l * alpha
            else:
                acc = acc * alpha[:, None]
                l = l * alpha
            m_ref = mnew
            l = l + p.sum(-1)
            acc = acc + p @ lat[j0:min(s1, j0 + BLK)]
            if mistake == "after_block":
                acc = acc * alpha[:, None]
        parts.append((acc, m_ref, l))
    M = np.max([p[1] for p in parts], axis=0)
    wts = [np.where(np.isfinite(p[1]), np.exp2(np.where(np.isfinite(p[1]), p[1] - M, 0.0)), 0.0) for p in parts]
    L = sum(wt * p[2] for wt, p in zip(wts, parts))
    return sum((wt / L)[:, None] * p[0] for wt, p in zip(wts, parts))


@pytest.mark.parametrize("mode,S", [("sparse", 2), ("dense", 4), ("sparse", 1)])
def test_rescale_mistakes_detected(mode, S):
    w, ref = _ref(mode, S)
    k = ref["scores"].shape[2]
    cache = w.cache.double().numpy()
    for b in range(w.B):
        if w.indices is None:
            pos = np.arange(k)
        else:
            pos = w.indices[b].numpy().astype(np.int64)
        lat = np.where((pos >= 0)[:, None], cache[b, np.clip(pos, 0, None), :workload.DC], 0.0)
        good = _lazy_mix(ref["scores"][b], lat, S)
        assert rel_err(good, ref["o_lat"][b]) <= 1e-9
    errs = {}
    for mistake in ("no_factor", "sum_only", "natural_units", "after_block"):
        worst = 0.0
        for b in range(w.B):
            pos = np.arange(k) if w.indices is None else w.indices[b].numpy().astype(np.int64)
            lat = np.where((pos >= 0)[:, None], cache[b, np.clip(pos, 0, None), :workload.DC], 0.0)
            worst = max(worst, rel_err(_lazy_mix(ref["scores"][b], lat, S, mistake), ref["o_lat"][b]))
        errs[mistake] = worst
    assert all(e > REL_TOL for e in errs.values()), errs
