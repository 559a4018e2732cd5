#!/usr/bin/env python3
"""Throughput of CompactFusion's fused residual-compression + error-feedback step on
one MI355X, on the FLUX-shaped sequence-parallel shard.

Workload (synthetic stand-in for FLUX.1-dev activations, see ``gen``): 114 tensors per
denoising step (57 layers x K,V), each 1024 tokens x 3072 channels bf16, per-channel
lognormal scales with 1% outlier channels x20, drift 0.05 per step, 28 steps; step 0 is
the warmup (the activation itself is sent), the rest are Compact-1bit compressed.

A timed "step" compresses all 114 tensors of one denoising step with error feedback,
as one C-ABI call over the step's slab (the tensors laid out back to back), inputs
resident in HBM.  The per-layer pattern (57 calls of K and V) is reported beside it.
``value`` is GB/s of bf16 input activation (2 B x elements / time).  The JSON line also
carries the roofline of the compress kernel (algorithmic bytes per launch / average
launch time from HIP events around every launch), the oracle timed on the host cores
on a bounded sample, and the other rows of the path (2-bit, decode, warmup init,
CogVideoX-shaped shard) measured in the same process.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compress+EF GB/s of bf16 activation per GPU; % of HBM peak (FLUX shard)"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
MFMA_FP32_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
# algorithmic bytes per element: a (bf16) read, ahat read + write, err write, codes, scales
BYTES_PER_ELEM = {
    "compress1": 2 + 4 + 4 + 4 + 1 / 8 + 4 / 128,
    "compress2": 2 + 4 + 4 + 4 + 2 / 8 + 4 / 128,
    "decode1": 4 + 4 + 1 / 8 + 4 / 128,
    "decode2": 4 + 4 + 2 / 8 + 4 / 128,
    "decode2_bf16": 4 + 4 + 2 + 2 / 8 + 4 / 128,  # plus the bf16 copy for the attention consumer
    "init": 2 + 4 + 4,
    # top-k sender: the quantizer's 14 B of state traffic, then k index bytes and k bf16
    # values per group; receiver: the payload and one read + write of the mirror (k
    # scattered 4-byte updates per group touch most 64-byte sectors anyway)
    "topk12": 2 + 4 + 4 + 4 + 12 * 3 / 128,
    "topk6": 2 + 4 + 4 + 4 + 6 * 3 / 128,
    "topk_decode12": 4 + 4 + 12 * 3 / 128,
    # senders without the (diagnostic) error buffer: no 4-byte e write per element
    "compress1_noerr": 2 + 4 + 4 + 1 / 8 + 4 / 128,
    "topk12_noerr": 2 + 4 + 4 + 12 * 3 / 128,
}


def lowrank_fused(m: int, rank: int) -> bool:
    """Whether the library runs the iterations after the first as one fused pass over r
    (back-projection and the next projection together): for m <= 1024 rows and a rank
    padded to 16 of at most 32.  The kernel list of a profiled call shows k_lr_backfore
    exactly when this holds."""
    return m <= 1024 and (rank + 15) // 16 * 16 <= 32


def lowrank_bytes_per_elem(iters: int, fused: bool = False) -> float:
    """Algorithmic HBM bytes per element of one low-rank step: the first projection
    reads a and Ahat and writes r (10 B), each further projection and each
    back-projection reads r (4 B), the reconstruction reads a and Ahat and writes
    Ahat and e (14 B).  With the fused pass a back-projection and the next projection
    read r once, so r is read iters + 1 times in all instead of 2 iters."""
    reads = iters + 1 if fused else 2 * iters
    return 10 + 4 * (reads - 1) + 14


def lowrank_flops_per_elem(rank: int, iters: int) -> float:
    """Algorithmic flops per element: 2k per projection and per back-projection pass,
    2k for the reconstruction."""
    return 4 * rank * iters + 2 * rank
# the headline kernel's sources: its own file and the device helpers it includes
KERNEL_SRCS = [os.path.join(ROOT, "activation_residual_compression_cf_amd", "csrc", f)
               for f in ("cf_quant.hip", "cf_vec.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "compress_q1_flux_pmc.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None when the
    kernel source changed since the counters were taken."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != kernel_hash():
        return None
    return float(b.group(1))


def call_times(torch, fn, reps, warm=1):
    """ms of each of reps back-to-back calls of fn(), each bracketed by events, after
    `warm` untimed calls (the first launch of a kernel also loads its code object)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return [x.elapsed_time(y) for x, y in pairs]


def time_calls(torch, fn, reps, warm=1):
    """Mean ms per call of fn() over reps back-to-back calls."""
    ts = call_times(torch, fn, reps, warm)
    return sum(ts) / len(ts)


def cpu_baseline(wl, host_steps, bits, threads):
    """The oracle, as it stands, on the host cores: full compressed steps of all tensors,
    one tensor per task."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from gen import as_f32, start_basis

    gen_f32 = lambda x: as_f32(x).astype(np.float32).copy()
    O = oracle.default()
    S = wl.slots
    ahat = np.empty((S, wl.m, wl.n), np.float32)
    err = np.empty_like(ahat)
    for s in range(S):
        O.init_state(host_steps[0][s], ahat[s], err[s])
    nsteps = len(host_steps) - 1

    def task(args):
        t, s = args
        O.compress(bits, host_steps[t][s], ahat[s], err[s])

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for t in range(1, nsteps + 1):
            list(ex.map(task, [(t, s) for s in range(S)]))
    dt = time.perf_counter() - t0
    elems = nsteps * S * wl.m * wl.n
    # single-thread figure on one tensor
    a1 = np.empty((wl.m, wl.n), np.float32)
    e1 = np.empty_like(a1)
    O.init_state(host_steps[0][0], a1, e1)
    t1 = time.perf_counter()
    O.compress(bits, host_steps[1][0], a1, e1)
    dt1 = time.perf_counter() - t1
    # low rank: one tensor, one compressed step, single thread, per configuration
    lowrank = {}
    for rank, iters in ((32, 2), (8, 10)):
        ah = gen_f32(host_steps[0][0])
        er = np.zeros_like(ah)
        q = start_basis(0, 0, wl.n, rank).copy()
        t2 = time.perf_counter()
        O.lowrank_compress(np.ascontiguousarray(host_steps[1][0]), ah, er, q, rank, iters, 4)
        dt2 = time.perf_counter() - t2
        lowrank[f"r{rank}_q{iters}_int4"] = {"ms_per_tensor": round(dt2 * 1e3, 1),
                                             "GBs": round(wl.m * wl.n * 2 / dt2 / 1e9, 5)}
    import gen as _gen

    avail = _gen.affinity_cores()
    return {
        "value": round(elems * 2 / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "cores_available": avail,
        "thread_cap": None if threads == avail else
        f"{threads} worker threads: the host CPU share of one GPU, of {avail} cores the process may use",
        "kind": "oracle",
        "sample": f"{nsteps} compressed steps x {S} tensors of {wl.m}x{wl.n} bf16 "
                  f"(Compact-{bits}bit, one tensor per task, {threads} threads), {dt:.2f} s wall, "
                  f"{dt * threads:.1f} thread-seconds",
        "single_thread_GBs": round(wl.m * wl.n * 2 / dt1 / 1e9, 4),
        "lowrank_single_thread": lowrank,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25, help="timed denoising steps")
    ap.add_argument("--warmup", type=int, default=2, help="untimed compressed steps")
    ap.add_argument("--per-call", type=int, default=114,
                    help="tensors per C-ABI call (114 = the whole step as one slab; 2 = one "
                         "layer's K,V)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the secondary rows")
    ap.add_argument("--rows", default="",
                    help="comma-separated name prefixes of the secondary rows to run (default all)")
    ap.add_argument("--repeats", type=int, default=3,
                    help="whole-trajectory repeats timed after the headline steps (0: none)")
    ap.add_argument("--no-kernel-times", action="store_true",
                    help="skip the profiled pass that times each low-rank kernel (for runs under rocprofv3)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also launch one plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the compressor works on one sequence-parallel "
              "rank's shard with no inter-GPU traffic; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    from activation_residual_compression_cf_amd import cf

    dev = cf.require_device()
    wl = gen.WORKLOADS["flux"]
    numel = wl.numel
    bits = 1
    n_gen = wl.steps  # the whole trajectory: the timed steps, then the repeats over all of it
    log(f"generating {n_gen} steps of {wl.slots} x {wl.m}x{wl.n} bf16 on the host")
    t0 = time.perf_counter()
    tr = gen.Trajectory(wl, args.seed)
    steps_d = []
    host_keep = []
    n_host = 4  # steps kept on the host for the oracle baseline (3 compressed: ~25 s of CPU work)
    for t in range(n_gen):
        a = tr.next()
        if t < n_host:
            host_keep.append(a.copy())
        steps_d.append(torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16))
    torch.cuda.synchronize()
    log(f"generated and uploaded in {time.perf_counter() - t0:.1f} s")

    slab = cf.Slab(wl.slots, numel, bits, dev)
    slab.init(steps_d[0], args.per_call)
    compressed = list(range(1, n_gen))

    def step_input(i):
        return steps_d[compressed[i % len(compressed)]]

    for i in range(args.warmup):
        slab.compress(step_input(i), args.per_call)
    torch.cuda.synchronize()

    # timed region: K steps bracketed by HIP events on the launch stream
    per_call = max(1, min(args.per_call, wl.slots))
    calls_per_step = -(-wl.slots // per_call)

    def stamp():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start = stamp()
    marks = [start]
    for i in range(args.steps):
        slab.compress(step_input(args.warmup + i), per_call)
        marks.append(stamp())
    end = marks[-1]
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = start.elapsed_time(end)
    step_ms = sorted(x.elapsed_time(y) for x, y in zip(marks, marks[1:]))
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    ms_per_step = total_ms / args.steps
    step_bytes_act = wl.slots * numel * 2
    value = step_bytes_act / (ms_per_step / 1e3) / 1e9

    # average launch duration over the timed region (launches are back to back on
    # one stream; with one call per step this is the kernel's own duration)
    n_launch = args.steps * calls_per_step
    avg_launch_ms = total_ms / n_launch
    launch_elems = per_call * numel
    algo_bytes = launch_elems * BYTES_PER_ELEM["compress1"]
    achieved = algo_bytes / (avg_launch_ms / 1e3) / 1e9
    # the committed counters were taken on the whole-step launch (114 tensors per call)
    traffic = counter_traffic() if per_call == wl.slots else None
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": "k_compress<1, bf16> (one wave instruction per stream per 2-group tile, one-wave blocks in runs of 256 per XCD)",
        "algorithmic_bytes_per_launch": int(algo_bytes),
        "avg_launch_us": round(avg_launch_ms * 1e3, 2),
        "launches_timed": n_launch,
    }
    log(f"compress1 step {ms_per_step:.3f} ms, {value:.1f} GB/s act, launch {avg_launch_ms*1e3:.1f} us "
        f"-> {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of HBM), wall {wall:.3f} s")

    trajectory = trajectory_repeats(torch, slab, steps_d, per_call, args.repeats) if args.repeats else None

    rows = {}
    if not args.no_rows:
        want = [w for w in args.rows.split(",") if w]
        rows = secondary_rows(torch, np, cf, gen, dev, wl, steps_d, compressed, per_call, want,
                              kernel_times_on=not args.no_kernel_times)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")

    cpu = None
    if not args.no_cpu_baseline:
        threads = gen.default_threads()
        log(f"oracle baseline on {threads} host threads")
        cpu = cpu_baseline(wl, host_keep, bits, threads)
        log(f"oracle: {cpu['value']} GB/s ({cpu['sample']})")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(median_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "FLUX-shaped shard, Compact-1bit: 114 tensors/step (57 layers x K,V) of "
                        "1024 tokens x 3072 channels bf16, 28 steps, 1 warmup step",
            "tensors_per_step": wl.slots,
            "tokens": wl.m,
            "channels": wl.n,
            "bits": bits,
            "group": 128,
            "tensors_per_call": per_call,
            "calls_per_step": calls_per_step,
            "hbm_fraction_of_step": round(value * BYTES_PER_ELEM["compress1"] / 2 / HBM_PEAK_GBS, 4),
        },
        "roofline": roofline,
        "trajectory": trajectory,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


def _median(x):
    x = sorted(x)
    h = len(x) // 2
    return x[h] if len(x) % 2 else 0.5 * (x[h - 1] + x[h])


def trajectory_repeats(torch, slab, steps_d, per_call, repeats):
    """The headline step over the whole trajectory, `repeats` times: warmup step 0, then
    every compressed step once, each bracketed by events; per repeat and over all of
    them, the mean and median step time."""
    per_rep = []
    for _ in range(repeats):
        slab.init(steps_d[0], per_call)
        torch.cuda.synchronize()
        marks = []
        for t in range(1, len(steps_d)):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append(e)
            slab.compress(steps_d[t], per_call)
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        marks.append(e)
        torch.cuda.synchronize()
        per_rep.append([a.elapsed_time(b) for a, b in zip(marks, marks[1:])])
    flat = [x for r in per_rep for x in r]
    out = {"repeats": repeats, "compressed_steps_per_repeat": len(per_rep[0]),
           "ms_per_step_mean": round(sum(flat) / len(flat), 4), "ms_per_step_median": round(_median(flat), 4),
           "per_repeat_mean": [round(sum(r) / len(r), 4) for r in per_rep],
           "per_repeat_median": [round(_median(r), 4) for r in per_rep]}
    log(f"trajectory x{repeats}: mean {out['ms_per_step_mean']} ms, median {out['ms_per_step_median']} ms per step")
    return out


def secondary_rows(torch, np, cf, gen, dev, wl, steps_d, compressed, per_call, want=(), kernel_times_on=True):
    """The other rows of the path, each timed with events over whole steps.  `want`
    selects rows by name prefix (all when empty)."""
    numel = wl.numel
    rows = {}
    step_elems = wl.slots * numel

    def on(name):
        # a row runs when a wanted prefix matches it; a group gate also runs when the
        # wanted prefix names one of its rows
        return not want or any(name.startswith(w) or w.startswith(name) for w in want)

    def row(name, ms, bytes_key, elems=step_elems):
        gbs_act = elems * 2 / (ms / 1e3) / 1e9
        hbm = elems * BYTES_PER_ELEM[bytes_key] / (ms / 1e3) / 1e9
        rows[name] = {"ms_per_step": round(ms, 4), "act_GBs": round(gbs_act, 1),
                      "hbm_GBs": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBS, 4)}
        log(f"{name}: {ms:.3f} ms/step, {gbs_act:.0f} GB/s act, {hbm / HBM_PEAK_GBS:.1%} of HBM")

    # 2-bit compress on the same shard, its receiver decode, 1-bit decode and init
    if on("compress2_flux") or on("decode") or on("init"):
        quant_rows(torch, cf, dev, wl, steps_d, compressed, per_call, row, on)
    if on("compress1_flux_per_layer"):
        per_layer_row(torch, cf, dev, wl, steps_d, compressed, row)
    if on("lowrank"):
        lowrank_rows(torch, np, cf, gen, dev, wl, steps_d, compressed, rows, step_elems, on, kernel_times_on)
    if on("topk"):
        topk_rows(torch, cf, dev, wl, steps_d, compressed, row, on)
    if on("noerr"):
        noerr_rows(torch, np, cf, gen, dev, wl, steps_d, compressed, row, rows, step_elems)
    if on("compress2_cogvideo"):
        cogvideo_row(torch, np, cf, gen, dev, per_call, row)
    if on("ef_study"):
        rows["ef_study_flux_1bit"] = ef_study(torch, cf, wl, steps_d)
    if on("lowrank_study"):
        rows["lowrank_study_flux"] = lowrank_study(torch, np, cf, gen, wl, steps_d)
    if on("sparse_study"):
        rows["sparse_study_flux"] = sparse_study(torch, cf, wl, steps_d)
    torch.cuda.empty_cache()
    return rows


def quant_rows(torch, cf, dev, wl, steps_d, compressed, per_call, row, on):
    numel = wl.numel
    s2 = cf.Slab(wl.slots, numel, 2, dev)
    s2.init(steps_d[0], per_call)
    s2.compress(steps_d[compressed[0]], per_call)
    it = iter(range(10 ** 9))
    ms = time_calls(torch, lambda: s2.compress(steps_d[compressed[(next(it) + 1) % len(compressed)]],
                                               per_call), 8)
    row("compress2_flux", ms, "compress2")
    # receiver decode, 1-bit and 2-bit (from the sender's last payload)
    for bits, src in ((2, s2),):
        rx = cf.Slab(wl.slots, numel, bits, dev, receiver=True)
        rx.init(steps_d[0], per_call)
        ms = time_calls(torch, lambda: rx.decompress(src.codes, src.scales, per_call), 8)
        row(f"decode{bits}_flux", ms, f"decode{bits}")
        # the same decode with the bf16 copy of the reconstruction, as one call for the step
        out16 = torch.empty(wl.slots * numel, dtype=torch.bfloat16, device=dev)
        rxf, cf_, sf_ = rx.ahat.view(-1), src.codes.view(-1), src.scales.view(-1)
        ms = time_calls(torch, lambda: cf.decompress(bits, cf_, sf_, rxf, out_bf16=out16), 8)
        row(f"decode{bits}_bf16_flux", ms, f"decode{bits}_bf16")
        del rx, out16
    s1 = cf.Slab(wl.slots, numel, 1, dev)
    s1.init(steps_d[0], per_call)
    s1.compress(steps_d[compressed[0]], per_call)
    rx = cf.Slab(wl.slots, numel, 1, dev, receiver=True)
    rx.init(steps_d[0], per_call)
    ms = time_calls(torch, lambda: rx.decompress(s1.codes, s1.scales, per_call), 8)
    row("decode1_flux", ms, "decode1")
    ms = time_calls(torch, lambda: s1.init(steps_d[0], per_call), 8)
    row("init_flux", ms, "init")
    del s1, s2, rx


def topk_rows(torch, cf, dev, wl, steps_d, compressed, row, on):
    """Top-k sparsifier on the whole step in one call: k = 12 (the 2-bit byte budget) and
    k = 6 (about the 1-bit budget), and the k = 12 receiver decode."""
    n = wl.slots * wl.numel
    ahat = torch.empty(n, dtype=torch.float32, device=dev)
    err = torch.empty_like(ahat)
    for k in (12, 6):
        if not on(f"topk{k}_flux"):
            continue
        idx = torch.empty(n // 128 * k, dtype=torch.uint8, device=dev)
        vals = torch.empty(n // 128 * k, dtype=torch.int16, device=dev)
        cf.init_state(steps_d[0], ahat, err)
        it = iter(range(10 ** 9))
        ms = time_calls(torch, lambda: cf.topk_compress(
            k, steps_d[compressed[next(it) % len(compressed)]].reshape(-1), ahat, err, idx, vals), 8)
        row(f"topk{k}_flux", ms, f"topk{k}")
        if k == 12 and on("topk12_decode_flux"):
            rx = ahat.clone()
            ms = time_calls(torch, lambda: cf.topk_decompress(k, idx, vals, rx), 8)
            row("topk12_decode_flux", ms, "topk_decode12")
            del rx
        del idx, vals
    del ahat, err
    torch.cuda.empty_cache()


def noerr_rows(torch, np, cf, gen, dev, wl, steps_d, compressed, row, rows, step_elems):
    """The senders with err = NULL (the error feedback lives in ahat; the error buffer is
    diagnostic): 1-bit and top-12 over the whole step, and low rank r32/q2."""
    n = wl.slots * wl.numel
    ahat = torch.empty(n, dtype=torch.float32, device=dev)
    cf.init_state(steps_d[0], ahat)
    codes = torch.empty(n // 8, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 128, dtype=torch.float32, device=dev)
    it = iter(range(10 ** 9))
    ms = time_calls(torch, lambda: cf.compress(1, steps_d[compressed[next(it) % len(compressed)]].reshape(-1),
                                               ahat, None, codes, scales), 8)
    row("noerr_compress1_flux", ms, "compress1_noerr")
    idx = torch.empty(n // 128 * 12, dtype=torch.uint8, device=dev)
    vals = torch.empty(n // 128 * 12, dtype=torch.int16, device=dev)
    cf.init_state(steps_d[0], ahat)
    ms = time_calls(torch, lambda: cf.topk_compress(12, steps_d[compressed[next(it) % len(compressed)]].reshape(-1),
                                                    ahat, None, idx, vals), 8)
    row("noerr_topk12_flux", ms, "topk12_noerr")
    del codes, scales, idx, vals
    rank, iters = 32, 2
    ah3 = ahat.view(wl.slots, wl.m, wl.n)
    cf.init_state(steps_d[0], ah3)
    qs = torch.from_numpy(np.stack([gen.start_basis(0, s, wl.n, rank) for s in range(wl.slots)])).to(dev)
    ws = torch.empty(cf.lowrank_workspace_bytes(wl.m, wl.n, rank, wl.slots), dtype=torch.uint8, device=dev)
    pay = cf.lowrank_payload(wl.slots, wl.m, wl.n, rank, 4, dev)
    a3 = [steps_d[c].view(wl.slots, wl.m, wl.n) for c in compressed]
    ms = time_calls(torch, lambda: cf.lowrank_compress(a3[next(it) % len(a3)], ah3, None, qs, rank, iters, 4,
                                                       pay, ws), 4)
    # the reconstruction reads ahat only and writes ahat
    bpe = lowrank_bytes_per_elem(iters, lowrank_fused(wl.m, rank)) - 6
    hbm = step_elems * bpe / (ms / 1e3) / 1e9
    rows["noerr_lowrank_r32_q2_int4_flux"] = {"ms_per_step": round(ms, 4), "hbm_GBs": round(hbm, 1),
                                               "hbm_frac": round(hbm / HBM_PEAK_GBS, 4), "bytes_per_elem": bpe}
    log(f"noerr_lowrank_r32_q2_int4_flux: {ms:.3f} ms/step, {hbm / HBM_PEAK_GBS:.1%} of HBM")
    del ahat, qs, ws, pay
    torch.cuda.empty_cache()


def per_layer_row(torch, cf, dev, wl, steps_d, compressed, row):
    """Per-layer pattern: 57 back-to-back calls of one layer's K and V."""
    numel = wl.numel
    s1 = cf.Slab(wl.slots, numel, 1, dev)
    s1.init(steps_d[0], 2)
    it2 = iter(range(10 ** 9))
    ms = time_calls(torch, lambda: s1.compress(steps_d[compressed[next(it2) % len(compressed)]],
                                               2), 8)
    row("compress1_flux_per_layer", ms, "compress1")
    # the same 57 calls captured once per input step in a HIP graph and replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    for j in range(4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            s1.compress(steps_d[compressed[j % len(compressed)]], 2)
        graphs.append(g)
    torch.cuda.synchronize()
    it3 = iter(range(10 ** 9))
    ms = time_calls(torch, lambda: graphs[next(it3) % len(graphs)].replay(), 8)
    row("compress1_flux_per_layer_graph", ms, "compress1")
    # the same 57 calls alternating over two streams: consecutive layers' calls are
    # independent, so one call's ramp and drain overlap the next call's streaming
    pair = [torch.cuda.Stream(), torch.cuda.Stream()]
    it4 = iter(range(10 ** 9))

    def two_streams():
        cur = torch.cuda.current_stream()
        for x in pair:
            x.wait_stream(cur)
        s1.compress(steps_d[compressed[next(it4) % len(compressed)]], 2, streams=pair)
        for x in pair:
            cur.wait_stream(x)

    ms = time_calls(torch, two_streams, 8)
    row("compress1_flux_per_layer_2streams", ms, "compress1")
    # and that fork and join captured in a HIP graph (two parallel branches) and replayed
    graphs = []
    for j in range(4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            cur = torch.cuda.current_stream()
            for x in pair:
                x.wait_stream(cur)
            s1.compress(steps_d[compressed[j % len(compressed)]], 2, streams=pair)
            for x in pair:
                cur.wait_stream(x)
        graphs.append(g)
    torch.cuda.synchronize()
    it5 = iter(range(10 ** 9))
    ms = time_calls(torch, lambda: graphs[next(it5) % len(graphs)].replay(), 8)
    row("compress1_flux_per_layer_2streams_graph", ms, "compress1")
    del graphs, s1
    torch.cuda.empty_cache()


def kernel_times(torch, fn, reps=3):
    """Device time per call of each low-rank kernel that fn() launches, from a separate
    profiled pass of `reps` calls (torch.profiler, which on ROCm reads the kernel records
    of the HIP runtime's tracer), in microseconds, keyed by kernel name.  None when the
    profiler cannot record device activity here."""
    try:
        from torch.profiler import ProfilerActivity, profile

        fn()
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
        out = {}
        for ev in prof.key_averages():
            m = re.search(r"k_lr_([a-z]+)(ILb1E|<true)?", ev.key)
            if not m:
                continue
            name = "k_lr_" + m.group(1) + ("<first>" if m.group(1) == "project" and m.group(2) else "")
            t = getattr(ev, "device_time_total", None)
            if t is None:
                t = getattr(ev, "cuda_time_total", 0.0)
            out[name] = round(out.get(name, 0.0) + t / reps, 1)
        return out or None
    except Exception as exc:  # noqa: BLE001 - the profiler is optional here
        log(f"kernel_times: profiler unavailable ({type(exc).__name__}: {exc})")
        return None


def lowrank_rows(torch, np, cf, gen, dev, wl, steps_d, compressed, rows, step_elems, on, kernel_times_on=True):
    """Compact-Lowrank on the FLUX shard: one call per step over all 114 tensors."""
    for rank, iters in ((32, 2), (8, 10)):
        if not on(f"lowrank_r{rank}_q{iters}"):
            continue
        ahat = torch.empty((wl.slots, wl.m, wl.n), dtype=torch.float32, device=dev)
        err = torch.empty_like(ahat)
        cf.init_state(steps_d[0], ahat, err)
        qs = torch.from_numpy(np.stack([gen.start_basis(0, s, wl.n, rank)
                                        for s in range(wl.slots)])).to(dev)
        ws = torch.empty(cf.lowrank_workspace_bytes(wl.m, wl.n, rank, wl.slots), dtype=torch.uint8,
                         device=dev)
        pay = cf.lowrank_payload(wl.slots, wl.m, wl.n, rank, 4, dev)
        a3 = [steps_d[c].view(wl.slots, wl.m, wl.n) for c in compressed]
        cf.lowrank_compress(a3[0], ahat, err, qs, rank, iters, 4, pay, ws)
        it4 = iter(range(10 ** 9))
        ts = call_times(torch, lambda: cf.lowrank_compress(a3[1 + next(it4) % (len(a3) - 1)], ahat,
                                                           err, qs, rank, iters, 4, pay, ws), 8)
        ms = sum(ts) / len(ts)
        fused = lowrank_fused(wl.m, rank)
        bpe = lowrank_bytes_per_elem(iters, fused)
        fpe = lowrank_flops_per_elem(rank, iters)
        hbm = step_elems * bpe / (ms / 1e3) / 1e9
        name = f"lowrank_r{rank}_q{iters}_int4_flux"
        rows[name] = {"ms_per_step": round(ms, 4), "ms_per_step_median": round(_median(ts), 4),
                      "act_GBs": round(step_elems * 2 / (ms / 1e3) / 1e9, 1),
                      "hbm_GBs": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBS, 4),
                      "tflops": round(step_elems * fpe / (ms / 1e3) / 1e12, 2),
                      "mfma_fp32_frac": round(step_elems * fpe / (ms / 1e3) / 1e12 / MFMA_FP32_TFLOPS, 4),
                      "bytes_per_elem": bpe, "fused_pass": fused,
                      "bytes_per_elem_unfused": lowrank_bytes_per_elem(iters), "flops_per_elem": fpe,
                      "payload_bytes_per_tensor": wl.m * rank // 2 + wl.n * rank // 2 + 8 * rank}
        log(f"{name}: {ms:.3f} ms/step (median {_median(ts):.3f}), {hbm / HBM_PEAK_GBS:.1%} of HBM, "
            f"{rows[name]['tflops']} TFLOP/s")
        kt = kernel_times(torch, lambda: cf.lowrank_compress(a3[1 + next(it4) % (len(a3) - 1)], ahat, err, qs, rank,
                                                             iters, 4, pay, ws)) if kernel_times_on else None
        rows[name]["kernel_us_per_call"] = kt
        if kt and ("k_lr_backfore" in kt) != fused:
            log(f"{name}: the profiled kernels disagree with the fused-pass rule ({sorted(kt)})")
            rows[name]["fused_rule_mismatch"] = True
        if kt:
            orth = sum(v for k, v in kt.items() if k in ("k_lr_gram", "k_lr_solve"))
            rows[name]["orth_us_per_call"] = round(orth, 1)
            rows[name]["orth_us_per_iteration"] = round(orth / iters, 1)
            log(f"{name}: kernels (us per call) {kt}; orth {orth:.1f} us per call")
        rx = torch.empty_like(ahat)
        cf.init_state(steps_d[0], rx)
        ms = time_calls(torch, lambda: cf.lowrank_decompress(4, pay, rx, rank), 4)
        rows[f"lowrank_r{rank}_decode_flux"] = {"ms_per_step": round(ms, 4),
                                               "hbm_frac": round(step_elems * 8 / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        del ahat, err, qs, ws, pay, rx
        torch.cuda.empty_cache()


def ef_study(torch, cf, wl, steps_d):
    """Error-feedback study on the FLUX trajectory (all tensors, Compact-1bit): the
    relative error ||A_t - Ahat_t|| / ||A_t - A_{t-1}|| with error feedback, without it
    (quantized raw step deltas), and for naive 1-bit of the whole activation."""
    n = wl.slots * wl.numel
    dev = steps_d[0].device
    ef = cf.SenderState.create(n, dev)
    cf.init_state(steps_d[0], ef.ahat, ef.err)
    mirror = torch.empty(n, dtype=torch.float32, device=dev)
    cf.init_state(steps_d[0], mirror)
    naive = torch.empty(n, dtype=torch.float32, device=dev)
    codes = torch.empty(n // 8, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 128, dtype=torch.float32, device=dev)
    out = {"steps": [], "ef": [], "no_ef": [], "naive": []}
    for t in range(1, len(steps_d)):
        a = steps_d[t].reshape(-1)
        cf.compress(1, a, ef.ahat, ef.err, codes, scales)
        cf.compress_ablation(cf.CF_MODE_NOEF, 1, a, mirror, a_prev=steps_d[t - 1].reshape(-1),
                             codes=codes, scales=scales)
        cf.compress_ablation(cf.CF_MODE_NAIVE, 1, a, naive, codes=codes, scales=scales)
        if t in (1, 2, 4, 8, 16, len(steps_d) - 1):
            a32 = a.float()
            step = torch.linalg.norm(a32 - steps_d[t - 1].reshape(-1).float()).item()
            out["steps"].append(t)
            out["ef"].append(round(torch.linalg.norm(a32 - ef.ahat).item() / step, 4))
            out["no_ef"].append(round(torch.linalg.norm(a32 - mirror).item() / step, 4))
            out["naive"].append(round(torch.linalg.norm(a32 - naive).item() / step, 4))
            del a32
    log(f"ef_study: ||A-Ahat||/||dA|| at steps {out['steps']}: EF {out['ef']}, "
        f"no EF {out['no_ef']}, naive {out['naive']}")
    del ef, mirror, naive
    torch.cuda.empty_cache()
    return out


def sparse_study(torch, cf, wl, steps_d):
    """Top-k against the quantizers at equal bytes on the FLUX trajectory (all tensors,
    error feedback on): ||A_t - Ahat_t|| / ||A_t - A_{t-1}|| for 1-bit (20 B per group)
    beside top-6 (18 B), and 2-bit (36 B) beside top-12 (36 B)."""
    n = wl.slots * wl.numel
    dev = steps_d[0].device
    arms = {"q1": 1, "top6": 6, "q2": 2, "top12": 12}
    st = {}
    for name in arms:
        s = cf.SenderState.create(n, dev)
        cf.init_state(steps_d[0], s.ahat, s.err)
        st[name] = s
    codes = torch.empty(n // 4, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 128, dtype=torch.float32, device=dev)
    idx = torch.empty(n // 128 * 12, dtype=torch.uint8, device=dev)
    vals = torch.empty(n // 128 * 12, dtype=torch.int16, device=dev)
    out = {"steps": [], **{k: [] for k in arms}}
    for t in range(1, len(steps_d)):
        a = steps_d[t].reshape(-1)
        for name, p in arms.items():
            s = st[name]
            if name.startswith("q"):
                cf.compress(p, a, s.ahat, s.err, codes[: n * p // 8], scales)
            else:
                cf.topk_compress(p, a, s.ahat, s.err, idx[: n // 128 * p], vals[: n // 128 * p])
        if t in (1, 2, 4, 8, 16, len(steps_d) - 1):
            a32 = a.float()
            step = torch.linalg.norm(a32 - steps_d[t - 1].reshape(-1).float()).item()
            out["steps"].append(t)
            for name in arms:
                out[name].append(round(torch.linalg.norm(a32 - st[name].ahat).item() / step, 4))
            del a32
    log("sparse_study: ||A-Ahat||/||dA|| at steps " + str(out["steps"]) + ": " +
        ", ".join(f"{k} {out[k]}" for k in arms))
    del st, codes, scales, idx, vals
    torch.cuda.empty_cache()
    return out


def lowrank_study(torch, np, cf, gen, wl, steps_d, nslots=16):
    """Low-rank variants on the first `nslots` FLUX tensors over the whole trajectory:
    final ||A - Ahat|| / ||A||, payload bytes per tensor and time per call (all 114
    tensors) for rank 32 INT4 (Compact-Lowrank) and rank 8 bf16 ("Pure Lowrank") at 2
    and 10 iterations, warm-started from the previous step's Q or cold (a fresh
    random basis every step)."""
    dev = steps_d[0].device
    arms = [("r32_q2_int4_warm", 32, 2, 4, True), ("r8_q2_bf16_warm", 8, 2, 16, True),
            ("r8_q10_bf16_warm", 8, 10, 16, True), ("r8_q2_bf16_cold", 8, 2, 16, False)]
    out = {}
    for name, rank, iters, fb, warm in arms:
        ahat = torch.empty((nslots, wl.m, wl.n), dtype=torch.float32, device=dev)
        err = torch.empty_like(ahat)
        a = [s.reshape(wl.slots, wl.m, wl.n)[:nslots] for s in steps_d]
        cf.init_state(a[0], ahat, err)
        basis = lambda seed: torch.from_numpy(np.stack([gen.start_basis(seed, s, wl.n, rank)
                                                        for s in range(nslots)])).to(dev)
        qs = basis(0)
        ws = torch.empty(cf.lowrank_workspace_bytes(wl.m, wl.n, rank, nslots), dtype=torch.uint8,
                         device=dev)
        for t in range(1, len(a)):
            if not warm:
                qs = basis(t)
            cf.lowrank_compress(a[t], ahat, err, qs, rank, iters, fb, workspace=ws)
        a32 = a[-1].float()
        rel = (torch.linalg.norm(a32 - ahat) / torch.linalg.norm(a32)).item()
        payload = (wl.m + wl.n) * rank * fb // 8 + (8 * rank if fb == 4 else 0)
        out[name] = {"final_rel_err": round(rel, 5), "payload_bytes": payload,
                     "ratio": round(wl.numel * 2 / payload, 1)}
        del ahat, err, a32, ws
    # time per call over all tensors for the 16-bit arms (the INT4 arm is timed in its row)
    for name, rank, iters, fb, warm in arms[1:3]:
        ahat = torch.empty((wl.slots, wl.m, wl.n), dtype=torch.float32, device=dev)
        err = torch.empty_like(ahat)
        cf.init_state(steps_d[0], ahat, err)
        qs = torch.from_numpy(np.stack([gen.start_basis(0, s, wl.n, rank)
                                        for s in range(wl.slots)])).to(dev)
        ws = torch.empty(cf.lowrank_workspace_bytes(wl.m, wl.n, rank, wl.slots), dtype=torch.uint8,
                         device=dev)
        pay = cf.lowrank_payload(wl.slots, wl.m, wl.n, rank, fb, dev)
        a3 = [x.view(wl.slots, wl.m, wl.n) for x in steps_d[1:]]
        cf.lowrank_compress(a3[0], ahat, err, qs, rank, iters, fb, pay, ws)
        it = iter(range(10 ** 9))
        ms = time_calls(torch, lambda: cf.lowrank_compress(a3[1 + next(it) % (len(a3) - 1)], ahat, err,
                                                           qs, rank, iters, fb, pay, ws), 4)
        out[name]["ms_per_step_114"] = round(ms, 4)
        del ahat, err, qs, ws, pay
    torch.cuda.empty_cache()
    log("lowrank_study: " + ", ".join(f"{k} err {v['final_rel_err']} ({v['ratio']}x)" for k, v in out.items()))
    return out


def cogvideo_row(torch, np, cf, gen, dev, per_call, row):
    """CogVideoX-shaped shard, Compact-2bit."""
    cw = gen.WORKLOADS["cogvideo"]
    tr = gen.Trajectory(cw, 0)
    cs = [torch.from_numpy(tr.next().view(np.int16)).to(dev).view(torch.bfloat16) for _ in range(4)]
    sc = cf.Slab(cw.slots, cw.numel, 2, dev)
    sc.init(cs[0], per_call)
    sc.compress(cs[1], per_call)
    it3 = iter(range(10 ** 9))
    ms = time_calls(torch, lambda: sc.compress(cs[2 + next(it3) % 2], per_call), 8)
    row("compress2_cogvideo", ms, "compress2", cw.slots * cw.numel)
    del sc, cs


if __name__ == "__main__":
    main()
