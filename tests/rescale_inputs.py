"""Inputs that drive the online softmax's lazy rescale (not collected by pytest).

The decode keeps, per head and key split, a reference maximum that moves only
when a block of 32 keys beats it by more than 8 log2 units; the running sum
and the accumulators are then multiplied by 2^(old - new) ("Softmax" page,
formula for A: the normalisation is over all keys, so every earlier term has
to be brought to the new maximum).  With N(0, 1) inputs no block ever beats
the reference by that much, so these inputs plant rotary-key spikes.

Every head's rotary query gets a shared component along one of two rotary
dimensions (even heads dimension 0, odd heads dimension 1), and the rotary
keys of chosen index slots get a large value along that dimension, so their
scores rise by about 10 log2 units per level above the noise:
  even heads: level 1 at one key of block max(1, nb // 4), a lazy (no
              rescale) rise of about 4 log2 units at keys 12.. of block
              nb // 2, level 2 at one key of the split's last block;
  odd heads:  level 1 at four keys of block nb // 2.
Blocks are counted inside each key split (split s holds index slots
[s * chunk, (s + 1) * chunk)).  The other values are N(0, 1) / 4, so the
noise stays well below the 8-unit threshold.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from sparse_mla_amd import workload

BLK = 32
LOG2E = 1.0 / math.log(2.0)
THRESH = 8.0          # log2 units a block must gain before the reference moves
Q_SPIKE = 4.0         # shared rotary query component
LEVEL = 24.0          # rotary key value of one level (about +10 log2 units)


def split_chunk(k_max: int, S: int) -> int:
    """Index slots per split: ceil(k_max / S) rounded up to whole blocks (the
    rule mla_sparse_decode documents)."""
    c = -(-k_max // S)
    return -(-c // BLK) * BLK


def spike_workload(mode: str, S: int, mask_first_block: bool = True):
    """A small workload with planted score spikes, laid out for S splits.
    mode: "sparse" (B=3, L=3000, k=1000) or "dense" (B=2, L=1001)."""
    if mode == "sparse":
        w = workload.make("sparse_b32_l4096_k2048", B=3, L=3000, k=1000)
    else:
        w = workload.make("dense_p1000_b1", B=2, L=1001)
    # Quarter-size noise (a power-of-two scale keeps every value exact in bf16).
    w.q_nope = (w.q_nope.float() * 0.25).to(torch.bfloat16)
    qpe = w.q_pe.float() * 0.25
    qpe[:, :, 0::2, 0] = Q_SPIKE
    qpe[:, :, 1::2, 1] = Q_SPIKE
    w.q_pe = qpe.to(torch.bfloat16)
    cache = w.cache.float()
    cache[..., workload.DC:] *= 0.25
    k_max = w.k_max
    chunk = split_chunk(k_max, S)
    if w.indices is not None and mask_first_block:
        # A split whose first block is fully masked and whose later blocks are not.
        b, s = (0, 1) if S > 1 else (1, 0)
        w.indices[b, s * chunk: s * chunk + BLK] = -1
    for b in range(w.B):
        Lb = int(w.seq_lens[b])
        for s in range(S):
            s0 = s * chunk
            n = min(chunk, k_max - s0)
            if n <= 0:
                continue
            nb = -(-n // BLK)
            plan = [  # (rotary dim, block, keys, value)
                (0, max(1, nb // 4), [5], LEVEL),
                (0, nb // 2, list(range(12, 32)), 10.0),
                (0, nb - 1, [1], 2 * LEVEL),
                (1, nb // 2, [0, 1, 2, 3], LEVEL),
            ]
            for dim, blk, keys, val in plan:
                for kk in keys:
                    i = s0 + blk * BLK + kk
                    if i >= s0 + n:
                        continue
                    pos = i if w.indices is None else int(w.indices[b, i])
                    if 0 <= pos < Lb:
                        cache[b, pos, workload.DC + dim] = val
    w.cache = cache.to(torch.bfloat16)
    return w


def rescale_events(scores: np.ndarray, S: int, margin: float = 0.0):
    """The blocks at which the lazy rule moves the reference maximum with a
    nonzero accumulator (a rescale), per (b, h, split), from scores in natural
    units [B, H, k] (-inf for masked slots) laid out by index slot.  An event
    counts only when the block beats the reference by more than
    THRESH + margin; blocks within the margin of the threshold are reported
    separately as ambiguous.  Returns (events, ambiguous): lists of
    (b, h, s, block)."""
    B, H, k = scores.shape
    chunk = split_chunk(k, S)
    u = scores * LOG2E
    events, ambiguous = [], []
    for s in range(S):
        s0 = s * chunk
        s1 = min(k, s0 + chunk)
        if s1 <= s0:
            continue
        nb = -(-(s1 - s0) // BLK)
        bm = np.full((B, H, nb), -np.inf)
        for j in range(nb):
            bm[:, :, j] = u[:, :, s0 + j * BLK: min(s1, s0 + (j + 1) * BLK)].max(-1)
        for b in range(B):
            for h in range(H):
                ref = -np.inf
                for j in range(nb):
                    m = bm[b, h, j]
                    if m == -np.inf:
                        continue
                    if ref == -np.inf:
                        ref = m
                        continue
                    gain = m - ref
                    if abs(gain - THRESH) <= margin:
                        ambiguous.append((b, h, s, j))
                    if gain > THRESH:
                        if gain > THRESH + margin:
                            events.append((b, h, s, j))
                        ref = m
    return events, ambiguous
