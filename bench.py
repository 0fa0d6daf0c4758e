"""Benchmark of the absorbed sparse MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 1000] [--workload NAME]

One step = mla_absorb_q + mla_sparse_decode + (mla_combine + mla_value_up, as
the single fused mla_combine_value_up launch when the plan splits the keys)
over a batch of B single-token queries, all inputs resident in HBM.  Input sets are
rotated (distinct index sets, queries and weight copies; whole caches when they
are small) so that every cycle moves >= 1 GB and the 256 MB memory-side cache
cannot serve a repeated step.  Prints ONE JSON line.

The roofline entry is for the dominant kernel (the sparse decode): its
algorithmic bytes per launch (selected cache rows at 1152 B + 4 B per index)
over its mean launch time, from HIP events bracketing K decode launches
issued back to back on its stream over the same rotating input sets (their
absorbed queries computed beforehand; the throughput pass has no events
inside the steps, and an event pair around every launch would add ~3 us).
The line also carries the per-head-query rate (128 x queries/s), the
attention-only rate (B over the mean time of decode + the separate split
combine, K pairs back to back; value-up excluded), the per-step time of five
trials of the K rotated steps (the value is the first's) and their median, a
warm figure labelled as such (one input set every step), and the attainable
peaks measured on the same GPU (sparse_mla_amd/peaks.py: streaming read, the
decode's row gather on random rows, dense bf16 MFMA) with the decode's
fraction of them and the side of both ridges its intensity falls on.
The CPU baseline runs the fp64 oracle (oracle/, test infrastructure) on a
bounded sample of the same workload.

The default warm-up is long (1000 steps, tens of ms): for the first tens of
milliseconds of back-to-back steps the GPU runs the step about 10 % slower
than in steady state (20 warm-up steps: 71 us/step; 1000: 64.5 us/step at
B=64, k=2048), and a decode loop runs in steady state.
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
    ap.add_argument("--cpu-sample", type=int, default=None, help="sequences in the oracle sample")
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
    """R input sets of one workload.  Large caches are shared and only the
    index sets, queries and weights rotate; small caches rotate too."""
    spec = workload.SPECS[name]
    cache_bytes = spec.B * spec.L * ROW_BYTES
    base = workload.make(name, device="cpu", cache_device="cuda")
    sets = []
    for v in range(R):
        if v == 0:
            w = base
        else:
            shared = base.cache if cache_bytes > (1 << 28) else None
            w = workload.make(name, device="cpu", cache_device="cuda", variant=v, lens=base.seq_lens.cpu(),
                              cache=shared)
        dev = {}
        for key in ("q_nope", "q_pe", "wkv_b", "indices", "wkv_b_fp8", "wkv_b_scale", "seq_lens"):
            t = getattr(w, key)
            dev[key] = None if t is None else t.to("cuda")
        w.q_nope, w.q_pe, w.wkv_b, w.indices = dev["q_nope"], dev["q_pe"], dev["wkv_b"], dev["indices"]
        w.wkv_b_fp8, w.wkv_b_scale, w.seq_lens = dev["wkv_b_fp8"], dev["wkv_b_scale"], dev["seq_lens"]
        sets.append(w)
    return sets


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

    def step(w):
        mla.mla_absorb_q(w.q_nope, w.wkv_b, bufs.q_abs)
        mla.mla_sparse_decode(bufs.q_abs, w.q_pe, w.kv, w.pe, w.seq_lens, w.max_len, w.indices, w.scale,
                              bufs.num_splits, bufs.workspace, bufs.o_latent, bufs.lse,
                              k_max=k_max)
        if bufs.num_splits > 1:
            mla.mla_combine_value_up(bufs.workspace, B, bufs.num_splits, w.wkv_b, bufs.out, lse=bufs.lse)
        else:
            mla.mla_value_up(bufs.o_latent, w.wkv_b, bufs.out)

    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    # Pass 1 (throughput): K steps bracketed by two events, nothing inside --
    # an event pair around every decode launch adds ~5 us to each step.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(sets[i % R])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    # Four more trials of the same K rotated steps (pass 1 is the first); the
    # line's value stays pass 1's, the median of the five is reported beside it.
    trials = [ms_step]
    for _ in range(4):
        start.record(stream)
        for i in range(args.steps):
            step(sets[i % R])
        end.record(stream)
        torch.cuda.synchronize()
        trials.append(start.elapsed_time(end) / args.steps)
    # A warm figure, labelled as such: the same input set every step, so the
    # 256 MB memory-side cache can serve what the rotation keeps it from.
    start.record(stream)
    for i in range(args.steps):
        step(sets[0])
    end.record(stream)
    torch.cuda.synchronize()
    warm_ms = start.elapsed_time(end) / args.steps
    last_set = sets[0]  # bufs.out holds the output of the warm pass's last step
    # Pass 2 (kernel time for the roofline): K decode launches back to back on
    # the same stream, cycling the input sets (their absorbed queries computed
    # beforehand), bracketed by two HIP events.  An event pair around every
    # launch would add ~3 us to each; back to back, the mean includes the
    # short gap between consecutive launches and nothing else.
    qabs = [mla.mla_absorb_q(w.q_nope, w.wkv_b) for w in sets]

    def decode_only(i):
        w = sets[i % R]
        mla.mla_sparse_decode(qabs[i % R], w.q_pe, w.kv, w.pe, w.seq_lens, w.max_len, w.indices, w.scale,
                              bufs.num_splits, bufs.workspace, bufs.o_latent, bufs.lse, k_max=k_max)

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
        decode_only(i)
        if bufs.num_splits > 1:
            mla.mla_combine(bufs.workspace, B, bufs.num_splits, bufs.o_latent, lse=bufs.lse)

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
        log(f"output projection: {op_ms * 1e3:.2f} us ({oproj['achieved_GBps']:.0f} GB/s)")
        del ox, wos, oout
    log(f"{args.steps} steps: {ms_step * 1e3:.2f} us/step (wall {wall * 1e6 / args.steps:.2f} us), "
        f"median of 5 trials {sorted(trials)[2] * 1e3:.2f} us, warm (no rotation) {warm_ms * 1e3:.2f} us; "
        f"decode kernel {decode_ms * 1e3:.2f} us, decode + combine {attn_ms * 1e3:.2f} us; "
        f"plan splits={bufs.num_splits}")

    # Algorithmic work.
    if dense:
        keys = int(w0.seq_lens.sum().item())
        idx_bytes = 0
    else:
        keys = int((w0.indices >= 0).sum().item())
        idx_bytes = 4 * keys
    dec_bytes = keys * ROW_BYTES + idx_bytes
    dec_flops = keys * FLOP_PER_KEY
    step_bytes = dec_bytes + WEIGHT_BYTES + B * (Q_BYTES_PER_QUERY + O_BYTES_PER_QUERY)
    step_flops = dec_flops + B * 2 * (2 * 128 * 128 * 512)
    dec_gbs = dec_bytes / (decode_ms * 1e-3) / 1e9
    dec_tflops = dec_flops / (decode_ms * 1e-3) / 1e12
    step_roof_s = max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (BF16_PEAK_TFLOPS * 1e12))

    # Sampled parity of the last full step's output against the oracle.
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
        log(f"oracle CPU baseline on {n_seq} sequences ...")
        _, dt, threads, _ = cpu_baseline(w0, n_seq, torch, workload)
        cpu = {"value": n_seq / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
               "sample": f"{n_seq} of {B} sequences of input set 0 (all 128 heads, all their selected "
                         f"positions), fp64 C oracle with OpenMP, {dt:.2f} s wall"}
        log(f"oracle: {dt:.2f} s for {n_seq} queries on {threads} threads")

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
            "workload": name, "B": B, "k_max": k_max, "selected_keys": keys,
            "cache": f"[{B}, {spec.L}, 576] bf16 packed rows", "rotating_sets": R,
            "num_splits": bufs.num_splits,
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
        "median_of_5_us_per_step": sorted(trials)[2] * 1e3,
        "warm_no_rotation": {"value": B / (warm_ms * 1e-3), "unit": "queries/s", "us_per_step": warm_ms * 1e3,
                             "note": "input set 0 every step (cache-warm; not the headline)"},
        "attention_only": {"value": B / (attn_ms * 1e-3), "unit": "queries/s", "us": attn_ms * 1e3,
                           "kernels": "mla_sparse_decode + mla_combine" if bufs.num_splits > 1
                           else "mla_sparse_decode"},
        "output_proj": oproj,
        "attainable": attain,
        "parity_sampled_rel_err": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
