"""Benchmark of the absorbed sparse MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 1000] [--workload NAME]

One step = mla_absorb_q + mla_sparse_decode + (mla_combine + mla_value_up, as
the single fused mla_combine_value_up launch when the plan splits the keys)
over a batch of B single-token queries, all inputs resident in HBM.  Input
sets are rotated, each with its own lengths, index sets, queries, weights and
whole cache, so that every cycle moves >= 1 GB of distinct bytes (printed)
and the 256 MB memory-side cache cannot serve a repeated step.  Each step's C
calls are made with arguments marshalled once per input set
(binding.StepLauncher).  Prints ONE JSON line.

`value` and `ms_per_step` come from the median of five trials of K rotated
steps, each bracketed by two HIP events with nothing recorded inside; the
five trials and the host's enqueue time per step in each are listed.

The roofline entry is for the dominant kernel (the sparse decode): its
algorithmic bytes per launch (selected cache rows at 1152 B + 4 B per index)
over its mean launch time, from HIP events bracketing K decode launches
issued back to back on its stream over the same rotating input sets (their
absorbed queries computed beforehand).
The line also carries the per-head-query rate (128 x queries/s), the
attention-only rate (B over the mean time of decode + the separate split
combine, K pairs back to back; value-up excluded), a warm figure labelled as
such (one input set every step), and the attainable peaks measured on the
same GPU (sparse_mla_amd/peaks.py: streaming read, the decode's row gather on
random rows, dense bf16 MFMA) with the decode's fraction of them and the side
of both ridges its intensity falls on.
Timed apart from the step and not part of `value`: the sparse prefill
(MFMA-bound, against the bf16 peak), the output projection after the step
(the call recommended at the batch first, the others beside it), the step
for 64, 32 and 16 heads, and, on the fp8 workload, the step reading the fp8
weight codes directly.
The CPU baseline runs the fp64 oracle (oracle/, test infrastructure) on a
bounded sample of the same workload.

The default warm-up is long (1000 steps, tens of ms), so that the timed
steps run in the GPU's steady state.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ROW_BYTES = 1152               # 512 latent + 64 rotary bf16 values per position
FLOP_PER_KEY = 2 * 128 * (576 + 512)
WEIGHT_BYTES = 2 * 128 * 128 * 512 * 2   # W_UK and W_UV, bf16
Q_BYTES_PER_QUERY = 128 * (128 + 64) * 2
O_BYTES_PER_QUERY = 128 * 128 * 2
HEADS = 128                    # query heads; one query = one sequence across all heads
METRIC = "sparse MLA decode queries/s at B=64,k=2048; % of HBM/MFMA roofline"
ROTATION = {"dense_p1000_b1": 32, "sparse_b32_l4096_k2048": 10, "longctx_b64_k2048": 6,
            "verylong_b128_l131072_k2048": 3, "dense_fp8w_b64_l8192": 2}


HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "sparse_mla_amd", "csrc", "mla_kernels.hip")


def counter_traffic(workload_name):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by a plain-copy calibration), or None when no
    record exists for this workload or the kernel source changed since."""
    import hashlib

    path = os.path.join(HERE, "profiles", f"decode_kernel_counters_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return float(rec["decode_kernel_hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default=None, help="workload name (default: the B=64, k=2048 long-context case)")
    ap.add_argument("--rotate", type=int, default=None, help="input sets cycled through (default per workload)")
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the attainable-peak microbenchmarks")
    ap.add_argument("--no-output-proj", action="store_true", help="skip timing the output projection")
    ap.add_argument("--no-prefill", action="store_true", help="skip timing the sparse prefill")
    ap.add_argument("--no-heads", action="store_true", help="skip timing the head-sharded steps")
    ap.add_argument("--cpu-sample", type=int, default=None, help="sequences per oracle call")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="timed oracle work of the CPU baseline (calls repeat over the input sets until then)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    return ap.parse_args()


def copy_calibration(torch):
    """Five plain 1 GiB device copies, each from its own source; the sources
    are filled in order first, so each has left the 256 MB memory-side cache
    before it is read and every read goes to HBM."""
    n = 1 << 30
    srcs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(5)]
    dst = torch.empty_like(srcs[0])
    torch.cuda.synchronize()
    for src in srcs:
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": {"read": n, "write": n}, "launches": len(srcs)}))


def make_sets(name, R, torch, workload):
    """R independent input sets of one workload: each draws its own lengths,
    index sets, queries, weights and whole cache (variant seeds), so no two
    sets share a selected row, a recent-token window or a weight byte."""
    sets = []
    for v in range(R):
        w = workload.make(name, device="cpu", cache_device="cuda", variant=v)
        dev = {}
        for key in ("q_nope", "q_pe", "wkv_b", "indices", "wkv_b_fp8", "wkv_b_scale", "seq_lens"):
            t = getattr(w, key)
            dev[key] = None if t is None else t.to("cuda")
        w.q_nope, w.q_pe, w.wkv_b, w.indices = dev["q_nope"], dev["q_pe"], dev["wkv_b"], dev["indices"]
        w.wkv_b_fp8, w.wkv_b_scale, w.seq_lens = dev["wkv_b_fp8"], dev["wkv_b_scale"], dev["seq_lens"]
        sets.append(w)
    return sets


def step_bytes_of(w, torch):
    """Algorithmic HBM bytes of one step over input set w: the selected rows,
    both weight slices, the queries, the outputs and the index lists."""
    if w.indices is None:
        keys = int(w.seq_lens.sum().item())
        idx_bytes = 0
    else:
        keys = int((w.indices >= 0).sum().item())
        idx_bytes = 4 * keys
    return keys, keys * ROW_BYTES + idx_bytes, keys * ROW_BYTES + idx_bytes + WEIGHT_BYTES + \
        w.B * (Q_BYTES_PER_QUERY + O_BYTES_PER_QUERY)


def prefill_pass(args, mla, workload, torch, stream):
    """The sparse prefill (mla_sparse_prefill) of one 4096-token prompt, each
    token selecting 2048 positions, timed on its own (not part of `value`):
    K launches back to back between two events.  One prompt's cache (4.7 MB)
    and the weights stay in the GPU's caches across launches: the prefill is
    bound by the matrix cores, not HBM, so no rotation is needed.  FLOPs are
    those the absorbed form executes (278 528 per attended key, plus absorb and
    value-up per token); the full-sequence MHA form of the pages would need
    81 920 per attended key plus the up-projection of every position."""
    cfg = workload.PREFILL_HEADLINE
    B, T, k = cfg["B"], cfg["T"], cfg["k"]
    p = workload.make_prefill(B, T, k, device="cpu", cache_device="cuda")
    q_nope, q_pe, wkv_b, idx = (p.q_nope.to("cuda"), p.q_pe.to("cuda"), p.wkv_b.to("cuda"), p.indices.to("cuda"))
    S = mla.mla_plan(B * T, k, False)
    ws = torch.empty(mla.mla_prefill_workspace_bytes(B, T, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, T, HEADS, 128), dtype=torch.bfloat16, device="cuda")

    def run():
        mla.mla_sparse_prefill(q_nope, q_pe, p.kv, p.pe, wkv_b, idx, p.scale, num_splits=S, workspace=ws, out=out)

    for _ in range(3):
        run()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(3, min(args.steps, 20))
    d0.record(stream)
    for _ in range(n):
        run()
    d1.record(stream)
    torch.cuda.synchronize()
    ms = d0.elapsed_time(d1) / n
    r = p.indices.long()
    s_pos = torch.arange(T)[None, :, None]
    keys = int(((r >= 0) & (r <= s_pos)).sum().item())
    tok_flops = 2 * (2 * 128 * 128 * 512)
    flops = keys * FLOP_PER_KEY + B * T * tok_flops
    mha_flops = keys * 2 * 128 * (192 + 128) + B * T * tok_flops
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"prefill B={B} T={T} k={k}: {ms * 1e3:.1f} us ({B * T / (ms * 1e-3):.0f} tokens/s, {tflops:.0f} TFLOP/s)")
    return {"workload": f"prefill_b{B}_t{T}_k{k}", "us": ms * 1e3, "tokens_per_s": B * T / (ms * 1e-3),
            "attended_keys": keys, "num_splits": S, "launches_timed": n,
            "bound": "mfma", "tflops": tflops, "peak_tflops": BF16_PEAK_TFLOPS, "mfma_frac": tflops / BF16_PEAK_TFLOPS,
            "flops_per_launch": flops, "flops_mha_form": mha_flops,
            "kernels": "mla_sparse_prefill (absorb + causal sparse attention + merge/value-up)"}


def cpu_baseline(w, n_seq, torch, workload):
    """The fp64 oracle on the first n_seq sequences of input set 0: selected
    rows are gathered to the host (marshalling, untimed), the oracle call is
    timed."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    rows = list(range(n_seq))
    kvs, pes, idxs, lens = [], [], [], []
    for b in rows:
        Lb = int(w.seq_lens[b])
        if w.indices is None:
            pos = torch.arange(Lb, device="cuda")
        else:
            pos = w.indices[b].long()
            pos = pos[pos >= 0]
        r = w.cache[b].index_select(0, pos).cpu()
        kvs.append(r[:, : workload.DC])
        pes.append(r[:, workload.DC:])
        lens.append(r.shape[0])
    k = max(lens)
    kv = torch.zeros((n_seq, k, workload.DC), dtype=torch.bfloat16)
    pe = torch.zeros((n_seq, k, workload.DR), dtype=torch.bfloat16)
    for i in range(n_seq):
        kv[i, : lens[i]] = kvs[i]
        pe[i, : lens[i]] = pes[i]
    seq = torch.tensor(lens, dtype=torch.int32)
    wkv = w.wkv_b.cpu()
    qn = w.q_nope[:n_seq].cpu()
    qp = w.q_pe[:n_seq].cpu()
    t0 = time.perf_counter()
    res = oracle.decode(qn, qp, kv, pe, wkv, seq, None, w.scale)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return res, dt, threads, np


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2
    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return 0

    from sparse_mla_amd import binding as mla
    from sparse_mla_amd import workload

    name = args.workload or workload.HEADLINE
    spec = workload.SPECS[name]
    R = args.rotate or ROTATION[name]
    log(f"workload {name}: {spec.description}; {R} rotating input sets")
    t0 = time.perf_counter()
    sets = make_sets(name, R, torch, workload)
    if spec.fp8:  # one-time set-up, untimed: dequantise each weight copy once
        for w in sets:
            w.wkv_b = mla.mla_dequant_wkv_b_fp8(w.wkv_b_fp8, w.wkv_b_scale)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")

    w0 = sets[0]
    B = w0.B
    dense = w0.indices is None
    k_max = w0.k_max
    bufs = mla.DecodeBuffers.allocate(B, k_max, dense, num_splits=args.splits)
    stream = torch.cuda.current_stream()
    # One step's three C calls per input set, their arguments marshalled once.
    launchers = [mla.StepLauncher(bufs, w.q_nope, w.q_pe, w.kv, w.pe, w.wkv_b, w.seq_lens, w.max_len, w.indices,
                                  w.scale) for w in sets]
    per_set = [step_bytes_of(w, torch) for w in sets]
    distinct_bytes = sum(p[2] for p in per_set)
    log(f"{distinct_bytes / 1e9:.2f} GB of distinct algorithmic bytes per rotation cycle of {R} sets")

    for i in range(args.warmup):
        launchers[i % R]()
    torch.cuda.synchronize()

    # Five trials of K rotated steps, each bracketed by two events with
    # nothing recorded inside (an event pair around every decode launch adds
    # ~5 us to each step); `value` is from the median trial.  The host time
    # to enqueue each trial's K steps is recorded beside it: when it is close
    # to the GPU time, the host's launch rate sets the pace.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    trials, enqueue = [], []
    for _ in range(5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            launchers[i % R]()
        end.record(stream)
        enqueue.append((time.perf_counter() - t0) / args.steps)
        torch.cuda.synchronize()
        trials.append(start.elapsed_time(end) / args.steps)
    ms_step = sorted(trials)[2]
    # A warm figure, labelled as such: the same input set every step, so the
    # 256 MB memory-side cache can serve what the rotation keeps it from.
    start.record(stream)
    for i in range(args.steps):
        launchers[0]()
    end.record(stream)
    torch.cuda.synchronize()
    warm_ms = start.elapsed_time(end) / args.steps
    last_set = sets[0]
    # Steady state, labelled as such: the same rotated steps run continuously
    # for at least 50 ms first (under sustained load the GPU runs a few
    # milliseconds fast, then ~10 % slow for about ten milliseconds, then
    # settles), then five trials of K steps without a pause between them.
    t_end = time.perf_counter() + 0.05
    i = 0
    while time.perf_counter() < t_end:
        launchers[i % R]()
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    ev[0].record(stream)
    for t in range(5):
        for i in range(args.steps):
            launchers[i % R]()
        ev[t + 1].record(stream)
    torch.cuda.synchronize()
    steady = [ev[t].elapsed_time(ev[t + 1]) / args.steps for t in range(5)]
    steady_ms = sorted(steady)[2]
    # Pass 2 (kernel time for the roofline): K decode launches back to back on
    # the same stream, cycling the input sets, bracketed by two HIP events.
    # An event pair around every launch would add ~3 us to each; back to
    # back, the mean includes the short gap between consecutive launches and
    # nothing else.
    def decode_only(i):
        launchers[i % R].decode()

    for i in range(min(args.warmup, 100)):
        decode_only(i)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for i in range(args.steps):
        decode_only(i)
    d1.record(stream)
    torch.cuda.synchronize()
    decode_ms = d0.elapsed_time(d1) / args.steps
    # Pass 3 (attention-only rate): the key splits' decode plus the separate
    # split combine that yields the normalised latent output and its LSE, K
    # pairs back to back; value-up is left out.
    def attention_only(i):
        launchers[i % R].decode()
        launchers[i % R].combine()

    for i in range(min(args.warmup, 100)):
        attention_only(i)
    d0.record(stream)
    for i in range(args.steps):
        attention_only(i)
    d1.record(stream)
    torch.cuda.synchronize()
    attn_ms = d0.elapsed_time(d1) / args.steps
    # The step after the path, timed on its own (not part of `value`): the
    # output projection of the B value-up outputs to the model width, K
    # launches back to back over three weight copies (705 MB, beyond the
    # memory-side cache), bracketed by two events.
    oproj = None
    if not args.no_output_proj:
        ox, _ = workload.output_proj_inputs(B, device="cuda")
        wos = [workload.output_proj_inputs(1, seed=700 + 2 * c, device="cuda")[1] for c in range(3)]
        oout = torch.empty((B, 1, mla.MODEL_DIM), dtype=torch.bfloat16, device="cuda")
        for i in range(6):
            mla.mla_output_proj(ox, wos[i % 3], oout)
        d0.record(stream)
        for i in range(args.steps):
            mla.mla_output_proj(ox, wos[i % 3], oout)
        d1.record(stream)
        torch.cuda.synchronize()
        op_ms = d0.elapsed_time(d1) / args.steps
        op_bytes = wos[0].numel() * 2 + B * (HEADS * 128 + mla.MODEL_DIM) * 2
        oproj = {"us": op_ms * 1e3, "bytes_per_launch": op_bytes, "achieved_GBps": op_bytes / (op_ms * 1e-3) / 1e9,
                 "frac_hbm": op_bytes / (op_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "tflops": 2.0 * B * HEADS * 128 * mla.MODEL_DIM / (op_ms * 1e-3) / 1e12,
                 "kernel": "mla_output_proj", "weights": "bf16 [7168, 16384], 3 rotated copies"}
        # The same launches on the repacked weight copies (one-time set-up,
        # untimed): each group of 28 weight rows read as one contiguous stream.
        wps = [mla.mla_output_proj_pack(w) for w in wos]
        for i in range(6):
            mla.mla_output_proj_packed(ox, wps[i % 3], oout)
        d0.record(stream)
        for i in range(args.steps):
            mla.mla_output_proj_packed(ox, wps[i % 3], oout)
        d1.record(stream)
        torch.cuda.synchronize()
        pk_ms = d0.elapsed_time(d1) / args.steps
        oproj["packed_weights"] = {"us": pk_ms * 1e3, "achieved_GBps": op_bytes / (pk_ms * 1e-3) / 1e9,
                                   "frac_hbm": op_bytes / (pk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                   "kernel": "mla_output_proj_packed (weight from mla_output_proj_pack)"}
        # The inputs split in four (mla_output_proj_split: fp32 partial sums
        # in a workspace, added by a second launch), on the plain weights.
        ows = torch.empty(mla.mla_output_proj_split_workspace_bytes(B), dtype=torch.uint8, device="cuda")
        for i in range(6):
            mla.mla_output_proj_split(ox, wos[i % 3], ows, oout)
        d0.record(stream)
        for i in range(args.steps):
            mla.mla_output_proj_split(ox, wos[i % 3], ows, oout)
        d1.record(stream)
        torch.cuda.synchronize()
        sp_ms = d0.elapsed_time(d1) / args.steps
        split = {"us": sp_ms * 1e3, "bytes_per_launch": op_bytes, "achieved_GBps": op_bytes / (sp_ms * 1e-3) / 1e9,
                 "frac_hbm": op_bytes / (sp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "tflops": 2.0 * B * HEADS * 128 * mla.MODEL_DIM / (sp_ms * 1e-3) / 1e12,
                 "kernel": "mla_output_proj_split (4 input quarters, then their sum)",
                 "weights": "bf16 [7168, 16384], 3 rotated copies"}
        log(f"output projection: {op_ms * 1e3:.2f} us ({oproj['achieved_GBps']:.0f} GB/s); "
            f"packed weight {pk_ms * 1e3:.2f} us; inputs split in four {sp_ms * 1e3:.2f} us")
        # The call the library recommends at this batch leads: the split from
        # 32 rows on, the single pass below; the others follow.
        if B >= 32:
            packed = oproj.pop("packed_weights")
            oproj = dict(split, single_pass=oproj, packed_weights=packed)
        else:
            oproj["split_inputs"] = split
        del ox, wos, wps, oout, ows
    # fp8 weights: the same rotated steps with absorb and value-up reading the
    # block-scaled fp8 weight directly (16.8 MB of codes per step instead of
    # the 33.5 MB bf16 copy the step above reads), five trials, median.
    fp8_direct = None
    if spec.fp8:
        fl = [mla.StepLauncher(bufs, w.q_nope, w.q_pe, w.kv, w.pe, None, w.seq_lens, w.max_len, w.indices, w.scale,
                               w_fp8=w.wkv_b_fp8, w_scale=w.wkv_b_scale) for w in sets]
        for i in range(min(args.warmup, 100)):
            fl[i % R]()
        ftr = []
        for _ in range(5):
            start.record(stream)
            for i in range(args.steps):
                fl[i % R]()
            end.record(stream)
            torch.cuda.synchronize()
            ftr.append(start.elapsed_time(end) / args.steps)
        fms = sorted(ftr)[2]
        fbytes = sum(per_set[i % R][2] for i in range(args.steps)) / args.steps - WEIGHT_BYTES + WEIGHT_BYTES // 2 + 4096
        fp8_direct = {"value": B / (fms * 1e-3), "unit": "queries/s", "us_per_step": fms * 1e3,
                      "trials_us_per_step": [t * 1e3 for t in ftr],
                      "step_roofline_frac": fbytes / (HBM_PEAK_GBS * 1e9) / (fms * 1e-3),
                      "weight_bytes_per_step": WEIGHT_BYTES // 2 + 4096,
                      "kernels": "mla_absorb_q_fp8 + mla_sparse_decode + mla_combine_value_up_fp8"}
        log(f"fp8 weights read directly: {fms * 1e3:.2f} us/step")
    # Head-sharded step (one GPU's share of 16, 32 or 64 heads, with its rows
    # of wkv_b): the same rotated inputs, five trials of K steps, median.
    heads_sharded = None
    if not args.no_heads and not spec.fp8:
        heads_sharded = {}
        for H in (64, 32, 16):
            hb = mla.DecodeBuffers.allocate(B, k_max, dense, num_splits=bufs.num_splits, heads=H)
            shards = [(w.q_nope[:, :, :H].contiguous(), w.q_pe[:, :, :H].contiguous(),
                       w.wkv_b[: H * 256].contiguous()) for w in sets]
            hl = [mla.StepLauncher(hb, qn, qp, w.kv, w.pe, wk, w.seq_lens, w.max_len, w.indices, w.scale)
                  for w, (qn, qp, wk) in zip(sets, shards)]
            for i in range(min(args.warmup, 100)):
                hl[i % R]()
            htr = []
            for _ in range(5):
                start.record(stream)
                for i in range(args.steps):
                    hl[i % R]()
                end.record(stream)
                torch.cuda.synchronize()
                htr.append(start.elapsed_time(end) / args.steps)
            hms = sorted(htr)[2]
            hbytes = (sum(per_set[i % R][1] for i in range(args.steps)) / args.steps + WEIGHT_BYTES * H // 128 +
                      B * (Q_BYTES_PER_QUERY + O_BYTES_PER_QUERY) * H // 128)
            heads_sharded[str(H)] = {"us_per_step": hms * 1e3, "queries_per_s": B / (hms * 1e-3),
                                     "trials_us_per_step": [t * 1e3 for t in htr],
                                     "step_roofline_frac": hbytes / (HBM_PEAK_GBS * 1e9) / (hms * 1e-3)}
            log(f"heads {H}: {hms * 1e3:.2f} us/step")
            del hl, shards, hb
    prefill = None
    if not args.no_prefill:
        prefill = prefill_pass(args, mla, workload, torch, stream)
    log(f"{args.steps} steps x 5 trials: " + ", ".join(f"{t * 1e3:.2f}" for t in trials) +
        f" us/step (median {ms_step * 1e3:.2f}); host enqueue " + ", ".join(f"{t * 1e6:.1f}" for t in enqueue) +
        f" us/step; steady state {steady_ms * 1e3:.2f} us; warm (no rotation) {warm_ms * 1e3:.2f} us; "
        f"decode kernel {decode_ms * 1e3:.2f} us, "
        f"decode + combine {attn_ms * 1e3:.2f} us; plan splits={bufs.num_splits}")

    # Algorithmic work per step: the mean over the K steps of a trial (step i
    # runs input set i % R; the decode pass cycles the sets the same way).
    keys = sum(per_set[i % R][0] for i in range(args.steps)) / args.steps
    dec_bytes = sum(per_set[i % R][1] for i in range(args.steps)) / args.steps
    step_bytes = sum(per_set[i % R][2] for i in range(args.steps)) / args.steps
    dec_flops = keys * FLOP_PER_KEY
    step_flops = dec_flops + B * 2 * (2 * 128 * 128 * 512)
    dec_gbs = dec_bytes / (decode_ms * 1e-3) / 1e9
    dec_tflops = dec_flops / (decode_ms * 1e-3) / 1e12
    step_roof_s = max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (BF16_PEAK_TFLOPS * 1e12))

    # Sampled parity of one full step's output against the oracle: input set
    # 0 once more, so that bufs.out is its output whatever ran last.
    launchers[0]()
    torch.cuda.synchronize()
    parity = None
    try:
        import numpy as np

        import oracle
        last = last_set
        b = 0
        Lb = int(last.seq_lens[b])
        pos = torch.arange(Lb, device="cuda") if dense else last.indices[b].long()
        pos = pos[pos >= 0]
        rows = last.cache[b].index_select(0, pos).cpu()[None]
        ref = oracle.decode(last.q_nope[:1].cpu(), last.q_pe[:1].cpu(), rows[..., : workload.DC],
                            rows[..., workload.DC:], last.wkv_b.cpu(), torch.tensor([rows.shape[1]]), None,
                            last.scale)["out"][0]
        got = bufs.out[0, 0].float().cpu().numpy()
        parity = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        log(f"sampled parity (sequence 0): max|O-O_ref|/max|O_ref| = {parity:.2e}")
    except Exception as e:  # noqa: BLE001 - report, do not hide the measurement
        log(f"sampled parity check skipped: {e!r}")

    # Attainable peaks on this machine (the second roofline column): a streaming
    # read, the decode's own row gather on random rows, dense bf16 MFMA.
    attain = None
    if not args.no_peaks:
        from sparse_mla_amd import peaks
        pk = peaks.measure()
        intensity = FLOP_PER_KEY / ROW_BYTES
        ridge_spec = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        ridge_meas = pk["mfma_bf16_TFLOPs"] * 1e12 / (pk["row_gather_GBps"] * 1e9)
        attain = dict(pk)
        if oproj is not None:
            oproj["frac_vs_stream_read"] = oproj["achieved_GBps"] / pk["stream_read_GBps"]
        attain.update({
            "decode_frac_vs_row_gather": dec_gbs / pk["row_gather_GBps"],
            "decode_mfma_frac_vs_measured": dec_tflops / pk["mfma_bf16_TFLOPs"],
            "intensity_flop_per_byte": intensity,
            "ridge_flop_per_byte": {"spec": ridge_spec, "measured": ridge_meas},
            "side_of_ridge": {"spec": "hbm" if intensity < ridge_spec else "mfma",
                              "measured": "hbm" if intensity < ridge_meas else "mfma"},
        })
        log(f"attainable: stream read {pk['stream_read_GBps']:.0f} GB/s (LDS-DMA {pk['stream_lds_dma_GBps']:.0f}), row gather {pk['row_gather_GBps']:.0f} GB/s, "
            f"bf16 MFMA {pk['mfma_bf16_TFLOPs']:.0f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        n_seq = args.cpu_sample or {"dense_p1000_b1": 1, "sparse_b32_l4096_k2048": 32, "longctx_b64_k2048": 64,
                                    "verylong_b128_l131072_k2048": 64, "dense_fp8w_b64_l8192": 8}[name]
        log(f"oracle CPU baseline on {n_seq} sequences per call, cycling the input sets ...")
        # Calls on the first n_seq sequences of each input set in turn until
        # about --cpu-seconds of timed oracle work (the gathers to the host
        # between calls are not timed).
        t_cpu, calls = 0.0, 0
        while calls == 0 or (t_cpu < args.cpu_seconds and calls < 1000):
            _, dt, threads, _ = cpu_baseline(sets[calls % R], n_seq, torch, workload)
            t_cpu += dt
            calls += 1
        sets_used = min(calls, R)
        cpu = {"value": calls * n_seq / t_cpu, "unit": "queries/s", "cores": threads, "kind": "oracle",
               "sample": f"{calls} calls on the first {n_seq} of {B} sequences of an input set ({sets_used} sets "
                         f"in turn; all 128 heads, all their selected positions), {calls * n_seq} queries, "
                         f"fp64 C oracle with OpenMP, {t_cpu:.1f} s of timed oracle work"}
        log(f"oracle: {t_cpu:.2f} s for {calls * n_seq} queries on {threads} threads")

    line = {
        "metric": METRIC,
        "value": B / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": name, "B": B, "k_max": k_max, "selected_keys_mean": keys,
            "cache": f"[{B}, {spec.L}, 576] bf16 packed rows, one per input set", "rotating_sets": R,
            "distinct_bytes_per_cycle": distinct_bytes, "num_splits": bufs.num_splits,
        },
        "roofline": {
            "bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS, "traffic": counter_traffic(name),
            "kernel": "mla_sparse_decode", "kernel_us": decode_ms * 1e3,
            "bytes_per_launch": dec_bytes, "mfma_tflops": dec_tflops,
            "mfma_frac": dec_tflops / BF16_PEAK_TFLOPS,
        },
        "step_roofline_frac": step_roof_s / (ms_step * 1e-3),
        "head_queries_per_s": HEADS * B / (ms_step * 1e-3),
        "trials_us_per_step": [t * 1e3 for t in trials],
        "value_from": "median of the 5 trials",
        "host_enqueue_us_per_step": [t * 1e6 for t in enqueue],
        "steady_state": {"value": B / (steady_ms * 1e-3), "unit": "queries/s", "us_per_step": steady_ms * 1e3,
                         "trials_us_per_step": [t * 1e3 for t in steady],
                         "note": "median of five trials of the same rotated steps after >= 50 ms of continuous steps"},
        "warm_no_rotation": {"value": B / (warm_ms * 1e-3), "unit": "queries/s", "us_per_step": warm_ms * 1e3,
                             "note": "input set 0 every step (cache-warm; not the headline)"},
        "attention_only": {"value": B / (attn_ms * 1e-3), "unit": "queries/s", "us": attn_ms * 1e3,
                           "kernels": "mla_sparse_decode + mla_combine" if bufs.num_splits > 1
                           else "mla_sparse_decode"},
        "output_proj": oproj,
        "prefill": prefill,
        "fp8_weights_direct": fp8_direct,
        "heads_sharded": heads_sharded,
        "attainable": attain,
        "parity_sampled_rel_err": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
