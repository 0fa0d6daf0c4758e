"""Seeded synthetic inputs for the absorbed sparse MLA decode step.

This module holds no arithmetic of the method: it only draws random tensors
with the shapes, distributions and index structure of the workloads, so that
both the HIP path and the CPU oracle can be fed the same inputs.

Shapes follow the decode-branch code excerpt on the "Query-key similarity"
page: q_nope [B,1,H,128], q_pe [B,1,H,64] (already rotated), a latent cache of
512 features and a rotary-key cache of 64 features per position, and wkv_b of
H*(128+128) rows by 512 columns.  Caches are stored packed, one 576-value row
per position (latent followed by rotary key); ``kv``/``pe`` are views into it.

Seeds: workload seed ``s``; tensor j draws from a generator seeded ``s + j``
(0 q_nope, 1 q_pe, 2 cache, 3 wkv_b, 4 lengths, 5 indices, 6 fp8 scales,
7 fp8 values).  ``variant`` v adds 100*v to every seed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

H, DN, DR, DC, DV = 128, 128, 64, 512, 128
DQK = DC + DR                 # 576 features per cached position
SOFTMAX_SCALE = (DN + DR) ** -0.5   # qk_head_dim ** -0.5 with qk_head_dim = 192


@dataclass(frozen=True)
class Spec:
    """A workload recipe.

    lens: "fixed" (every L_b = L) or "ragged" (L_b uniform in [lo, L]).
    select: "dense" (no index list: every position), "uniform" (k distinct
    positions uniformly without replacement) or "recent" (the most recent
    w = min(512, k/4) positions plus k-w drawn uniformly from the rest, in
    shuffled order; every position when L_b <= k).
    """
    name: str
    B: int
    L: int
    k: Optional[int]
    select: str
    lens: str = "fixed"
    lo: int = 0
    fp8: bool = False
    seed: int = 0
    description: str = ""


SPECS = {
    "dense_p1000_b1": Spec(
        "dense_p1000_b1", B=1, L=1001, k=None, select="dense", seed=1000,
        description="decode of position 1000: B=1, 1001 cached positions, all selected"),
    "sparse_b32_l4096_k2048": Spec(
        "sparse_b32_l4096_k2048", B=32, L=4096, k=2048, select="uniform", seed=2000,
        description="B=32, L=4096, k=2048 distinct positions uniform without replacement"),
    "longctx_b64_k2048": Spec(
        "longctx_b64_k2048", B=64, L=32768, k=2048, select="recent", lens="ragged",
        lo=2048, seed=3000,
        description="B=64, ragged L_b in [2048, 32768], k=2048: recent 512 + 1536 uniform"),
    "verylong_b128_l131072_k2048": Spec(
        "verylong_b128_l131072_k2048", B=128, L=131072, k=2048, select="uniform", seed=4000,
        description="B=128, L=131072 (19.3 GB cache), k=2048 uniform without replacement"),
    "dense_fp8w_b64_l8192": Spec(
        "dense_fp8w_b64_l8192", B=64, L=8192, k=None, select="dense", fp8=True, seed=5000,
        description="B=64, L=8192, all positions; wkv_b as fp8 e4m3 with 128x128 block scales"),
}
HEADLINE = "longctx_b64_k2048"


@dataclass
class Workload:
    spec: Spec
    B: int
    seq_lens: torch.Tensor            # int32 [B]
    max_len: int                      # max L_b
    q_nope: torch.Tensor              # bf16 [B,1,H,DN]
    q_pe: torch.Tensor                # bf16 [B,1,H,DR]
    cache: torch.Tensor               # bf16 [B, L_alloc, DQK] (latent | rotary)
    wkv_b: Optional[torch.Tensor]     # bf16 [H*(DN+DV), DC] (None when fp8)
    indices: Optional[torch.Tensor]   # int32 [B, k] or None (dense)
    wkv_b_fp8: Optional[torch.Tensor] = None    # uint8 codes [H*(DN+DV), DC]
    wkv_b_scale: Optional[torch.Tensor] = None  # fp32 [H*(DN+DV)/128, DC/128]
    scale: float = SOFTMAX_SCALE
    extra: dict = field(default_factory=dict)

    @property
    def kv(self) -> torch.Tensor:
        return self.cache[..., :DC]

    @property
    def pe(self) -> torch.Tensor:
        return self.cache[..., DC:]

    @property
    def k_max(self) -> int:
        return self.max_len if self.indices is None else int(self.indices.shape[1])


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal_bf16(shape, g, device, std: float = 1.0, chunk_rows: int = 1 << 16):
    """N(0, std^2) drawn in fp32 and rounded to bf16, generated in row chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, shape[-1]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1].copy_(x)
    return out


def _lengths(spec: Spec, B: int, L: int, seed: int) -> torch.Tensor:
    if spec.lens == "ragged":
        g = _gen("cpu", seed + 4)
        return torch.randint(spec.lo, L + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    return torch.full((B,), L, dtype=torch.int32)


def _indices(spec: Spec, lens: torch.Tensor, k: int, seed: int) -> torch.Tensor:
    g = _gen("cpu", seed + 5)
    rows = []
    for Lb in lens.tolist():
        if spec.select == "uniform":
            if Lb <= k:
                r = torch.randperm(Lb, generator=g)
            else:
                r = torch.randperm(Lb, generator=g)[:k]
        elif spec.select == "recent":
            if Lb <= k:
                r = torch.randperm(Lb, generator=g)
            else:
                w = min(512, k // 4)
                recent = torch.arange(Lb - w, Lb)
                rest = torch.randperm(Lb - w, generator=g)[: k - w]
                both = torch.cat([recent, rest])
                r = both[torch.randperm(k, generator=g)]
        else:
            raise ValueError(spec.select)
        if r.numel() < k:
            r = torch.cat([r, torch.full((k - r.numel(),), -1, dtype=r.dtype)])
        rows.append(r)
    return torch.stack(rows).to(torch.int32)


def fp8_weights(rows: int, cols: int, seed: int, device="cpu"):
    """fp8 E4M3FN codes and fp32 128x128 block scales: scales are 2^U(-8,-4);
    values are N(0,1) * scale^-1 * 512^-1/2 clipped to +-448 and rounded to
    e4m3 by torch's cast (round to nearest even)."""
    gs = _gen("cpu", seed + 6)
    scale = torch.exp2(torch.empty((rows // 128, cols // 128)).uniform_(-8.0, -4.0, generator=gs))
    gv = _gen("cpu", seed + 7)
    x = torch.randn((rows, cols), generator=gv, dtype=torch.float32)
    inv = (1.0 / scale).repeat_interleave(128, 0).repeat_interleave(128, 1)
    x = (x * inv * (DC ** -0.5)).clamp_(-448.0, 448.0)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.to(device), scale.to(torch.float32).to(device)


def make(name_or_spec, device="cpu", B: Optional[int] = None, L: Optional[int] = None,
         k: Optional[int] = None, variant: int = 0, lens: Optional[torch.Tensor] = None,
         cache_device=None, cache: Optional[torch.Tensor] = None) -> Workload:
    """Draw one workload.  B, L and k override the recipe (for small cases);
    ``cache_device`` lets the large cache be drawn on the GPU; ``cache`` reuses
    an existing cache tensor instead of drawing one."""
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    B = spec.B if B is None else B
    L = spec.L if L is None else L
    k = spec.k if k is None else k
    seed = spec.seed + 100 * variant
    cdev = device if cache_device is None else cache_device
    if lens is None:
        lens = _lengths(spec, B, L, seed)
    lens = lens.to(torch.int32)
    max_len = int(lens.max())
    q_nope = _normal_bf16((B, 1, H, DN), _gen(device, seed + 0), device)
    q_pe = _normal_bf16((B, 1, H, DR), _gen(device, seed + 1), device)
    if cache is None:
        cache = _normal_bf16((B, L, DQK), _gen(cdev, seed + 2), cdev)
    if spec.fp8:
        codes, sc = fp8_weights(H * (DN + DV), DC, seed, device)
        wkv_b = None
    else:
        codes = sc = None
        wkv_b = _normal_bf16((H * (DN + DV), DC), _gen(device, seed + 3), device, std=DC ** -0.5)
    idx = None
    if spec.select != "dense":
        idx = _indices(spec, lens, k, seed).to(device)
    return Workload(spec=spec, B=B, seq_lens=lens.to(device), max_len=max_len,
                    q_nope=q_nope, q_pe=q_pe, cache=cache, wkv_b=wkv_b, indices=idx,
                    wkv_b_fp8=codes, wkv_b_scale=sc)


def output_proj_inputs(B: int, seed: int = 607, device="cpu"):
    """Inputs of the output projection: head outputs x [B, 1, 128, 128] ~ N(0, 1)
    and the output weight wo [7168, 128 * 128] ~ N(0, 1/16384) (variance
    1/fan_in), bf16, drawn from generators seeded seed and seed + 1."""
    x = _normal_bf16((B, 1, H, DV), _gen(device, seed), device)
    wo = _normal_bf16((7168, H * DV), _gen(device, seed + 1), device, std=(H * DV) ** -0.5)
    return x, wo


@dataclass
class Prefill:
    """Inputs of a sparse prefill: B prompts of T tokens, each token with its
    own selection of k positions of its prompt."""
    B: int
    T: int
    q_nope: torch.Tensor              # bf16 [B, T, H, DN]
    q_pe: torch.Tensor                # bf16 [B, T, H, DR]
    cache: torch.Tensor               # bf16 [B, T, DQK] (latent | rotary) of the prompt positions
    wkv_b: torch.Tensor               # bf16 [H*(DN+DV), DC]
    indices: Optional[torch.Tensor]   # int32 [B, T, k] or None (every causal key)
    scale: float = SOFTMAX_SCALE

    @property
    def kv(self) -> torch.Tensor:
        return self.cache[..., :DC]

    @property
    def pe(self) -> torch.Tensor:
        return self.cache[..., DC:]


PREFILL_HEADLINE = dict(B=1, T=4096, k=2048)


def make_prefill(B: int, T: int, k: Optional[int], seed: int = 6000, device="cpu", cache_device=None) -> Prefill:
    """Seeded prefill inputs.  Token s selects, in shuffled order: while
    s + 1 <= k, every position 0 .. s and k - s - 1 later positions of the
    prompt (a top-k over causally masked index scores returns those too; the
    causal mask removes them), -1 where the prompt is shorter than k;
    otherwise the most recent min(512, k / 4) positions up to s and the rest
    uniformly without replacement from the earlier ones.  k=None: no index
    lists (every causal key).  Generators seeded seed + j as in make()."""
    cdev = device if cache_device is None else cache_device
    q_nope = _normal_bf16((B, T, H, DN), _gen(device, seed + 0), device)
    q_pe = _normal_bf16((B, T, H, DR), _gen(device, seed + 1), device)
    cache = _normal_bf16((B, T, DQK), _gen(cdev, seed + 2), cdev)
    wkv_b = _normal_bf16((H * (DN + DV), DC), _gen(device, seed + 3), device, std=DC ** -0.5)
    idx = None
    if k is not None:
        g = _gen("cpu", seed + 5)
        idx = torch.full((B, T, k), -1, dtype=torch.int32)
        recent = min(512, k // 4)
        for b in range(B):
            for s in range(T):
                if s + 1 <= k:
                    later = torch.randperm(T - s - 1, generator=g)[: k - s - 1] + s + 1
                    r = torch.cat([torch.arange(s + 1), later])
                else:
                    win = torch.arange(s + 1 - recent, s + 1)
                    rest = torch.randperm(s + 1 - recent, generator=g)[: k - recent]
                    r = torch.cat([win, rest])
                r = r[torch.randperm(r.numel(), generator=g)]
                idx[b, s, : r.numel()] = r.to(torch.int32)
        idx = idx.to(device)
    return Prefill(B=B, T=T, q_nope=q_nope, q_pe=q_pe, cache=cache, wkv_b=wkv_b, indices=idx)
