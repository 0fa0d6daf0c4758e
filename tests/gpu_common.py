"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_mla_amd import workload

# Target tolerance: max |O - O_ref| <= 1e-2 * max |O_ref| (the same bar is
# used for the absorbed query and the latent mix); softmax rows sum to one
# within 1e-3 (checked on the kernel's own scores and LSE, with the LSE itself
# held to the oracle's within lse_tol).
REL_TOL = 1e-2
ROWSUM_TOL = 1e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def to_gpu(w: workload.Workload) -> workload.Workload:
    dev = "cuda"
    mv = lambda t: None if t is None else t.to(dev)  # noqa: E731
    return workload.Workload(spec=w.spec, B=w.B, seq_lens=mv(w.seq_lens), max_len=w.max_len,
                             q_nope=mv(w.q_nope), q_pe=mv(w.q_pe), cache=mv(w.cache),
                             wkv_b=mv(w.wkv_b), indices=mv(w.indices), wkv_b_fp8=mv(w.wkv_b_fp8),
                             wkv_b_scale=mv(w.wkv_b_scale), scale=w.scale)


def oracle_ref(w: workload.Workload, rows=None, want_weights=False):
    """Oracle outputs for sequences ``rows`` (default all) of a CPU-side workload."""
    rows = list(range(w.B)) if rows is None else list(rows)
    sel = torch.tensor(rows)
    idx = None if w.indices is None else w.indices.cpu()[sel].to(torch.int64)
    if idx is None and want_weights:
        idx = torch.stack([torch.cat([torch.arange(int(w.seq_lens[r])),
                                      torch.full((w.max_len - int(w.seq_lens[r]),), -1)]) for r in rows])
    cache = w.cache.cpu()[sel]
    return oracle.decode(w.q_nope.cpu()[sel], w.q_pe.cpu()[sel], cache[..., :workload.DC],
                         cache[..., workload.DC:], w.wkv_b.cpu(), w.seq_lens.cpu()[sel], idx, w.scale,
                         want_weights=want_weights, want_attended=True, att_len=cache.shape[1])


def lse_bound(q_abs_ref, latents, scale: float) -> np.ndarray:
    """Per-(row, head) bound on |LSE_gpu - LSE_ref|, from oracle quantities only.

    The one rounding ahead of the scores is q~ to bf16 (the absorb output): a
    round-to-nearest bf16 value errs by at most 2^-9 of its magnitude, so the
    score of key t errs by at most scale * sum_c 2^-9 |q~_c| |c_t,c| (the
    rotary half is exact bf16 input).  LSE is a smooth maximum of the scores
    and moves by at most the largest score error.  The bound doubles that for
    the kernel's fp32 accumulation and adds 1e-5 for the LSE arithmetic.
    ``latents[i]`` holds the selected latent rows [n_i, 512] of row i."""
    qa = np.abs(np.asarray(q_abs_ref, dtype=np.float64))  # [rows, H, 512]
    tol = np.zeros(qa.shape[:2])
    for i, c in enumerate(latents):
        if len(c):
            tol[i] = scale * 2.0 ** -8 * (qa[i] @ np.abs(np.asarray(c, dtype=np.float64)).T).max(axis=1)
    return tol + 1e-5


def selected_latents(w: workload.Workload, rows=None):
    """The selected in-range latent rows of each sequence of a CPU-side workload."""
    rows = list(range(w.B)) if rows is None else list(rows)
    cache = w.cache.cpu()
    out = []
    for b in rows:
        L = int(w.seq_lens[b])
        if w.indices is None:
            pos = np.arange(L)
        else:
            idx = w.indices.cpu()[b].numpy()
            pos = np.unique(idx[(idx >= 0) & (idx < L)])
        out.append(cache[b, torch.from_numpy(pos), :workload.DC].double().numpy())
    return out


def lse_tol(w: workload.Workload, ref, rows=None) -> np.ndarray:
    return lse_bound(ref["q_abs"], selected_latents(w, rows), w.scale)


def lse_dev(lse_gpu: np.ndarray, ref) -> np.ndarray:
    """|LSE_gpu - LSE_ref| with equal infinities counting as zero."""
    a, r = np.asarray(lse_gpu, dtype=np.float64), np.asarray(ref["lse"], dtype=np.float64)
    same = (a == r)
    return np.where(same, 0.0, np.abs(a - r))


def rowsum_dev(ref_scores: np.ndarray, lse_gpu: np.ndarray) -> float:
    """max over (b,h) of |sum_t exp(s_ref[t] - LSE_gpu) - 1| over the selected slots
    (masked slots carry -inf and contribute 0)."""
    s = np.exp(ref_scores - lse_gpu[..., None])
    return float(np.max(np.abs(s.sum(-1) - 1.0)))


def gather_rows_for_oracle(w, rows):
    """Selected cache rows of sequences ``rows`` of a GPU-resident workload,
    compacted on the host (plumbing: torch index_select, no arithmetic), with
    the index lists remapped to 0..k-1.  Returns (kv, pe, lens, indices)."""
    kvs, pes, idxs, lens = [], [], [], []
    for b in rows:
        Lb = int(w.seq_lens[b])
        if w.indices is None:
            pos = torch.arange(Lb, device=w.cache.device)
            slot_pos = pos
        else:
            slot_pos = w.indices[b].long()
            pos = slot_pos[slot_pos >= 0]
        r = w.cache[b].index_select(0, pos).cpu()
        kvs.append(r[:, : workload.DC])
        pes.append(r[:, workload.DC:])
        lens.append(r.shape[0])
    k = max(lens)
    kv = torch.zeros((len(rows), k, workload.DC), dtype=torch.bfloat16)
    pe = torch.zeros((len(rows), k, workload.DR), dtype=torch.bfloat16)
    idx = torch.full((len(rows), k), -1, dtype=torch.int64)
    for i in range(len(rows)):
        kv[i, : lens[i]] = kvs[i]
        pe[i, : lens[i]] = pes[i]
        idx[i, : lens[i]] = torch.arange(lens[i])
    return kv, pe, torch.tensor(lens, dtype=torch.int32), idx
