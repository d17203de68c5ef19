#!/usr/bin/env python
"""KDA chunked-prefill forward benchmark (one MI355X).

A step is one pass of the whole hot path over one packed varlen batch:
chunk table -> gate cumsum + intra-chunk kernel -> recurrence + output
kernel.  It is issued as kda_chunk_intra followed by kda_chunk_recurrence
(the same kernels kda_chunk_fwd enqueues; the bench checks the two paths
agree bitwise).  Each kernel's duration is measured inside the timed region
with HIP events on the launch stream, on every EVENT_STRIDE-th step only: a
timing event costs ~3.5 us of stream time on this device, and three per
step would slow the very throughput being measured by ~10%.

Before the W warmup steps, untimed steps run for --settle-seconds of wall
time (default 0.3 s): this device takes tens of milliseconds of sustained
load to reach its steady clocks, and a 100-step window that starts after 20
warmup steps reads ~10% slower than one after 300 (110.9 vs 100.7 us per
headline step, measured back to back on one box).  The timed region is
still exactly K steps; the settle time and its step count are reported.

Inputs are resident in HBM before timing starts.  Several device copies of
the inputs are rotated so that every step reads inputs that are not left in
the 256 MB Infinity Cache by the previous step.

Prints ONE JSON line.  ``--gpus`` above 1 exits: the library runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s at T=8192,H=16,K=V=128 bf16; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, TFLOP/s
MALL_BYTES = 256 * 2**20
BLOCK_BYTES = 72192              # one (head, chunk) intermediate block
EVENT_STRIDE = 10                # steps between two that carry kernel events


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="untimed steps for this long before the warmup steps (device clocks)")
    ap.add_argument("--workload", default="headline",
                    help="headline | tiny | batchB | sharegpt | long")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies to rotate (0: enough to exceed 2x the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of the workload the oracle baseline runs (0: all)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until it has used this much CPU time")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter scale)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: per-config latency table (markdown)")
    ap.add_argument("--only", default="",
                    help="with --sweep: a comma-separated subset of the sweep's config names")
    return ap.parse_args()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on this workload with this kernel's current
    sources (its translation unit, the headers it includes, the flags)."""
    import re
    from chunked_kda_prefill_amd import build as kbuild
    path = os.path.join(ROOT, "profiles", "headline_hbm_traffic.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"<!-- traffic-json: (\{.*\}) -->", text)
    if not m:
        return None
    rec = json.loads(m.group(1))
    unit = kbuild.KERNEL_UNITS.get(kernel)
    if unit is None or rec.get("workload") != workload:
        return None
    k = rec.get(kernel)
    if k is None or k.get("kernel_hash") != kbuild.kernel_hash(unit):
        return None
    return int(round((k["fetch_kib"] * rec["fetch_factor"] + k["write_kib"] * rec["write_factor"]) * 1024))


SWEEP_CONFIGS = ["tiny", "headline"] + [f"batch{b}" for b in (1, 2, 4, 8, 16, 32, 64)] + \
    ["sharegpt", "long", "decode16x1_h12", "decode16x4_h12", "decode64x1_h16", "decode64x1_h96"]
# configs also timed through the fused-prologue entry points, and with the
# same prologue done by separate torch ops in front of the plain entry point
FUSED_SWEEP_CONFIGS = ("headline", "long", "decode16x1_h12", "decode16x4_h12", "decode64x1_h96")
# configs also timed with chunk-parallel state passing (kda_chunk_fwd_segmented)
# at these segment counts: the A/B of few, long chains
SEGMENT_SWEEP = {"batch1": (4, 8), "batch2": (4, 8), "long": (2, 4)}


def sweep(args, torch, np, kda, wl):
    """Per-config latency of one kda_chunk_fwd call on cold inputs: 20 warmup
    calls, then 100 calls, each after an untimed read of a 512 MiB device
    buffer that evicts L2 and the MALL (a read, so that no dirty lines are
    left to write back during the call), bracketed by HIP events on the
    call's stream.  The device copy that gives the bandwidth ceiling runs
    after --settle-seconds of copies.
    Prints a markdown table: median / p10 / p90, tokens/s, algorithmic GB/s
    and TFLOP/s, the fraction of 8 TB/s, and the fp64 oracle's rate on a
    bounded sample (a few heads) of the same inputs.  Decode configs are
    also timed through kda_decode_fwd; the FUSED_SWEEP_CONFIGS also through
    the fused-prologue entry points (raw q, k and strided bf16 beta logits),
    and with that prologue done by torch ops before the plain entry point;
    their decode configs also as a whole decode step with the gated RMSNorm
    (kda_decode_step_fused, and kda_decode_fwd_fused + kda_gated_rmsnorm)."""
    only = [x for x in args.only.split(",") if x]
    unknown = [x for x in only if x not in SWEEP_CONFIGS]
    if unknown:
        raise SystemExit(f"--only: not sweep configs: {unknown} (known: {SWEEP_CONFIGS})")
    configs = [n for n in SWEEP_CONFIGS if not only or n in only]
    import oracle
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    flush = torch.ones(128 * 2**20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    # achievable ceiling: a plain device copy of 1 GiB
    a = torch.ones(2**28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    # settle the device's clocks under load first (see --settle-seconds)
    t_settle = time.perf_counter() + max(0.0, args.settle_seconds)
    while True:
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        if time.perf_counter() >= t_settle:
            break
    def stream_gbs(fn, bytes_per_call):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 10 * bytes_per_call / (e0.elapsed_time(e1) * 1e-3) / 1e9
    nb = a.numel() * 4
    copy_gbs = stream_gbs(lambda: b.copy_(a), 2 * nb)            # the runtime's copy
    ew_gbs = stream_gbs(lambda: torch.mul(a, 1.0, out=b), 2 * nb)  # an elementwise kernel
    del a, b
    threads = oracle.max_threads()
    print(f"Device copy of 1 GiB (read + write): {copy_gbs:.0f} GB/s "
          f"({copy_gbs / HBM_PEAK_GBS:.1%} of 8 TB/s) through the runtime's copy, "
          f"{ew_gbs:.0f} GB/s ({ew_gbs / HBM_PEAK_GBS:.1%}) through an elementwise kernel "
          f"(x * 1). Oracle threads: {threads}.\n")
    print("| config | T | N | H | chunks | median µs | p10 µs | p90 µs | M tokens/s | GB/s | "
          "HBM frac | TFLOP/s | oracle tokens/s (heads) | GPU/oracle |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    runs = []
    for n in configs:
        main = ["decode_fwd", "chunk_fwd"] if n.startswith("decode") else ["chunk_fwd"]
        if n in FUSED_SWEEP_CONFIGS:
            main = main + [e + "_fused" for e in main] + ["torch prologue + " + main[0]]
            if n.startswith("decode"):
                main += ["decode_step_fused", "norm after decode_fwd_fused"]
        main += [f"segmented {p}" for p in SEGMENT_SWEEP.get(n, ())]
        runs += [(n, e) for e in main]
    for name, entry in runs:
        w = wl.by_name(name)
        T, N, H = w.T, w.N, w.H
        t = wl.to_torch(w, dev)
        ws = kda.new_workspace(T, N, H, dev)
        o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
        fin = torch.empty((N, H, 128, 128), dtype=torch.float32, device=dev)
        fused = "fused" in entry or "prologue" in entry
        step = entry in ("decode_step_fused", "norm after decode_fwd_fused")
        if fused:
            # raw q, k and bf16 beta logits in a strided [T, 5 + H + 3] slice
            rq, rk, bfull, pre = wl.raw_prologue_inputs(w, 300)
            bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(
                dev).view(torch.bfloat16)
            t["q"], t["k"], blog = bf(rq), bf(rk), bf(bfull)[:, pre:pre + H]
        if step:
            zfull = torch.randn((T, H * 128 + 128), device=dev).to(torch.bfloat16)
            z = zfull[:, 64:64 + H * 128].view(T, H, 128)
            nwt = torch.ones(128, dtype=torch.float32, device=dev)
            ybuf = torch.empty_like(o)
        is_dec = entry.split(" + ")[-1].startswith("decode_fwd")
        plain = kda.decode_fwd if is_dec else kda.chunk_fwd
        extra = {} if is_dec else {"workspace": ws}
        if entry.startswith("segmented"):
            nseg = int(entry.split()[1])
            sws = torch.empty(kda.load_library().kda_chunk_fwd_segmented_workspace_size(
                T, N, H, nseg), dtype=torch.uint8, device=dev)
            call = lambda: kda.chunk_fwd_segmented(
                t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], nseg,
                initial_state=t["initial_state"], scale=w.scale, o=o, final_state=fin,
                workspace=sws)
        elif entry == "decode_step_fused":
            call = lambda: kda.decode_step_fused(
                t["q"], t["k"], t["v"], t["g"], blog, t["cu_seqlens"], z, nwt,
                initial_state=t["initial_state"], scale=w.scale, o=o, y=ybuf, final_state=fin)
        elif entry == "norm after decode_fwd_fused":
            def call():
                kda.decode_fwd_fused(t["q"], t["k"], t["v"], t["g"], blog, t["cu_seqlens"],
                                     initial_state=t["initial_state"], scale=w.scale, o=o,
                                     final_state=fin)
                kda.gated_rmsnorm(o, z, nwt, out=ybuf)
        elif entry.endswith("_fused"):
            fn = kda.decode_fwd_fused if entry == "decode_fwd_fused" else kda.chunk_fwd_fused
            call = lambda: fn(t["q"], t["k"], t["v"], t["g"], blog, t["cu_seqlens"],
                              initial_state=t["initial_state"], scale=w.scale, qk_eps=1e-6,
                              o=o, final_state=fin, **extra)
        elif fused:
            def call():
                beta = torch.sigmoid(blog.float())
                qn = (t["q"].float() * torch.rsqrt((t["q"].float() ** 2).sum(-1, keepdim=True)
                                                   + 1e-6)).to(torch.bfloat16)
                kn = (t["k"].float() * torch.rsqrt((t["k"].float() ** 2).sum(-1, keepdim=True)
                                                   + 1e-6)).to(torch.bfloat16)
                plain(qn, kn, t["v"], t["g"], beta, t["cu_seqlens"],
                      initial_state=t["initial_state"], scale=w.scale, o=o, final_state=fin,
                      **extra)
        else:
            call = lambda: plain(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"],
                                 initial_state=t["initial_state"], scale=w.scale, o=o,
                                 final_state=fin, **extra)
        for _ in range(20):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(100)]
        for i, (x, y) in enumerate(evs):
            torch.sum(flush, dim=0, out=sink)
            x.record(stream)
            call()
            y.record(stream)
        torch.cuda.synchronize()
        us = np.array([x.elapsed_time(y) * 1e3 for x, y in evs])
        med, p10, p90 = (float(np.percentile(us, q)) for q in (50, 10, 90))
        nbytes, flops = wl.algorithmic_bytes(w), wl.algorithmic_flops(w)
        gbs = nbytes / (med * 1e-6) / 1e9
        # oracle on a bounded sample: at most 2 heads (tokens/s scaled to all)
        hs = list(range(min(H, 2)))
        c0 = time.perf_counter()
        oracle.kda_fwd(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.initial_state,
                       scale=w.scale, heads=hs)
        cw = time.perf_counter() - c0
        otps = T * len(hs) / H / cw
        label = w.name if entry == "chunk_fwd" else f"{w.name} ({entry.replace('_fwd', '')})"
        if step:
            del zfull, z, ybuf
        print(f"| {label} | {T} | {N} | {H} | {w.num_chunks()} | {med:.1f} | {p10:.1f} | "
              f"{p90:.1f} | {T / med:.2f} | {gbs:.0f} | {gbs / HBM_PEAK_GBS:.3f} | "
              f"{flops / (med * 1e-6) / 1e12:.1f} | {otps:,.0f} ({len(hs)}) | "
              f"{(T / (med * 1e-6)) / otps:,.0f}x |", flush=True)
        del t, ws, o, fin
        if fused:
            del blog
    norm_sweep(torch, np, kda, wl, dev, stream, flush, sink, configs)


def norm_sweep(torch, np, kda, wl, dev, stream, flush, sink, configs):
    """Cold latency of the gated-RMSNorm epilogue (kda_gated_rmsnorm) at the
    output shapes of FUSED_SWEEP_CONFIGS: x = o [T, H, 128] contiguous, the
    gate a column slice of a [T, H*128 + 128] bf16 tensor.  Algorithmic bytes
    per (token, head) row: 256 read of x, 256 of the gate, 256 written."""
    print("\n| epilogue config | T | H | median µs | p10 µs | p90 µs | GB/s | HBM frac |")
    print("|---|---|---|---|---|---|---|---|")
    for name in [n for n in FUSED_SWEEP_CONFIGS if n in configs]:
        w = wl.by_name(name)
        T, H = w.T, w.H
        x = torch.randn((T, H, 128), device=dev).to(torch.bfloat16)
        zf = torch.randn((T, H * 128 + 128), device=dev).to(torch.bfloat16)
        z = zf[:, 64:64 + H * 128].view(T, H, 128)
        wt = torch.ones(128, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(20):
            kda.gated_rmsnorm(x, z, wt, out=y)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(100)]
        for a, b in evs:
            torch.sum(flush, dim=0, out=sink)
            a.record(stream)
            kda.gated_rmsnorm(x, z, wt, out=y)
            b.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        med, p10, p90 = (float(np.percentile(us, q)) for q in (50, 10, 90))
        gbs = T * H * 768 / (med * 1e-6) / 1e9
        print(f"| {w.name} (gated_rmsnorm) | {T} | {H} | {med:.1f} | {p10:.1f} | {p90:.1f} | "
              f"{gbs:.0f} | {gbs / HBM_PEAK_GBS:.3f} |", flush=True)
        del x, zf, z, y


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs on one GPU only (asked for "
              f"{max(args.gpus, world)}); the KDA prefill path would shard by heads or by "
              "sequences, with no exchange inside the operation", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import chunked_kda_prefill_amd as kda
    from chunked_kda_prefill_amd import workloads as wl
    if args.sweep:
        sweep(args, torch, np, kda, wl)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.by_name(args.workload)
    T, N, H = w.T, w.N, w.H
    nc = w.num_chunks()

    if args.copy_calibration_mib > 0:
        nb = args.copy_calibration_mib * 2**20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    base = wl.to_torch(w, dev)
    in_bytes = sum(base[k].numel() * base[k].element_size()
                   for k in ("q", "k", "v", "g", "beta"))
    R = args.rotate if args.rotate > 0 else max(1, math.ceil(2 * MALL_BYTES / in_bytes) + 1)
    sets = [base] + [{k: (None if t is None else t.clone()) for k, t in base.items()}
                     for _ in range(R - 1)]
    o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((N, H, 128, 128), dtype=torch.float32, device=dev)
    ws = kda.new_workspace(T, N, H, dev)
    stream = torch.cuda.current_stream(dev)

    def step(s):
        kda.chunk_intra(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu_seqlens"],
                        scale=w.scale, workspace=ws)
        kda.chunk_recurrence(ws, T, N, H, initial_state=s["initial_state"], o=o,
                             final_state=fin)

    # the two-call step and the single kda_chunk_fwd call agree bitwise
    step(sets[0])
    o_ref, f_ref = kda.chunk_fwd(**{k: v for k, v in sets[0].items()}, scale=w.scale)
    torch.cuda.synchronize()
    same = bool(torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and
                torch.equal(fin, f_ref))
    if not same:
        raise SystemExit("bench.py: kda_chunk_fwd and intra+recurrence disagree")
    o_check = o.clone()
    f_check = fin.clone()
    del o_ref, f_ref

    # settle: untimed steps until the device has run under load for
    # --settle-seconds (its clocks reach their steady state), then W warmup steps
    settle_steps = 0
    t_settle = time.perf_counter() + max(0.0, args.settle_seconds)
    while time.perf_counter() < t_settle:
        for _ in range(10):
            step(sets[settle_steps % R])
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    # steps 5, 15, 25, ...: none right after the synchronize that starts the
    # timed region, whose first launch starts from an idle device
    sampled = list(range(min(EVENT_STRIDE // 2, args.steps - 1), args.steps, EVENT_STRIDE))
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = sets[i % R]
        e = ev.get(i)
        if e is not None:
            e[0].record(stream)
        kda.chunk_intra(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu_seqlens"],
                        scale=w.scale, workspace=ws)
        if e is not None:
            e[1].record(stream)
        kda.chunk_recurrence(ws, T, N, H, initial_state=s["initial_state"], o=o,
                             final_state=fin)
        if e is not None:
            e[2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    # step-time distribution: a separate, untimed pass with events around
    # every step (each event pair adds its own ~3.5 us to the interval)
    dist_n = max(10, min(50, args.steps))
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(dist_n)]
    for i, (ea, eb) in enumerate(dev_ev):
        ea.record(stream)
        step(sets[i % R])
        eb.record(stream)
    torch.cuda.synchronize()
    dist = np.array([ea.elapsed_time(eb) * 1e3 for ea, eb in dev_ev])
    step_dist = {"median": round(float(np.median(dist)), 2),
                 "p10": round(float(np.percentile(dist, 10)), 2),
                 "p90": round(float(np.percentile(dist, 90)), 2),
                 "from": f"{dist_n} further steps, each bracketed by HIP events "
                         "(not the timed region)"}
    ev = list(ev.values())
    intra_ms = [e[0].elapsed_time(e[1]) for e in ev]
    rec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    intra_us = 1e3 * float(np.mean(intra_ms))
    rec_us = 1e3 * float(np.mean(rec_ms))

    # --- algorithmic bytes / flops ---------------------------------------
    # Algorithmic bytes are what the operation must move: q, k, v, g, beta
    # read, o written (1,540 B per (token, head)), plus the initial and final
    # states.  The intermediate blocks the intra kernel writes and the
    # recurrence reads back are this design's own traffic, not the
    # operation's: they are reported separately (kernel_bytes_per_launch,
    # traffic_rate), never in `achieved`.
    path_bytes = wl.algorithmic_bytes(w)
    path_flops = wl.algorithmic_flops(w)
    blocks = nc * H
    h0_bytes = 0 if w.initial_state is None else N * H * 128 * 128 * 4
    intra_bytes = T * H * (3 * 256 + 512 + 4) + blocks * BLOCK_BYTES
    rec_bytes = blocks * BLOCK_BYTES + h0_bytes + T * H * 256 + N * H * 128 * 128 * 4
    kern = {"kda_intra": (intra_us, intra_bytes), "kda_recurrence": (rec_us, rec_bytes)}
    dom = max(kern, key=lambda k: kern[k][0])
    dom_us, dom_bytes = kern[dom]
    achieved = path_bytes / (dom_us * 1e-6) / 1e9
    step_s = elapsed / args.steps
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(w.name, dom),
                "achieved_from": "the path's algorithmic bytes (q, k, v, g, beta, o, states) "
                                 "per step / the dominant kernel's mean event time",
                "path_frac": round(path_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
                "kernel_us": {"kda_intra": round(intra_us, 2),
                              "kda_recurrence": round(rec_us, 2)},
                "kernel_us_from": f"HIP events on {len(ev)} of the {args.steps} timed steps "
                                  f"(every {EVENT_STRIDE}th, from step {sampled[0]})",
                "kernel_bytes_per_launch": {"kda_intra": intra_bytes,
                                            "kda_recurrence": rec_bytes},
                "traffic_rate": {k: round(b / (us * 1e-6) / 1e9, 1)
                                 for k, (us, b) in kern.items()},
                "traffic_rate_from": "kernel_bytes_per_launch (intermediate blocks included) "
                                     "/ mean event time, GB/s"}
    path = {"algorithmic_bytes": path_bytes, "algorithmic_flops": path_flops,
            "GB/s": round(path_bytes / step_s / 1e9, 1),
            "hbm_frac": round(path_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOP/s": round(path_flops / step_s / 1e12, 2),
            "mfma_frac": round(path_flops / step_s / 1e12 / BF16_PEAK_TFLOPS, 4),
            "step_us": step_dist}
    # secondary bounds: the path's bytes at 8 TB/s, its FLOP at the bf16 MFMA
    # peak, its exponentials (two per (token, head, key channel) in the intra
    # kernel) at the transcendental rate (a quarter of the fp32 lane rate:
    # 1,024 SIMDs x 4 per clock x 2.4 GHz), and the serial chain: the longest
    # (sequence, head) chain's chunk count and the recurrence time per chunk
    lens = np.diff(w.cu_seqlens.astype(np.int64))
    chain = int(((lens + 63) // 64).max()) if len(lens) else 0
    path["bounds_us"] = {
        "hbm": round(path_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
        "mfma_bf16": round(path_flops / (BF16_PEAK_TFLOPS * 1e12) * 1e6, 2),
        "transcendental": round(2 * T * H * 128 / (1024 * 4 * 2.4e9) * 1e6, 2),
        "chain_chunks": chain,
        "recurrence_us_per_chunk": round(rec_us / chain, 3) if chain else None}

    # --- CPU baseline: the fp64 oracle on a bounded sample -----------------
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        nh = H if args.cpu_heads <= 0 else min(args.cpu_heads, H)
        hsel = list(range(nh))
        threads = oracle.max_threads()
        walls = []
        cpu0 = time.process_time()
        while True:
            c0 = time.perf_counter()
            o_or, f_or = oracle.kda_fwd(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens,
                                        w.initial_state, scale=w.scale, heads=hsel)
            walls.append(time.perf_counter() - c0)
            if time.process_time() - cpu0 >= args.cpu_seconds or len(walls) >= 50:
                break
        cpu_s = time.process_time() - cpu0
        wall = float(np.median(walls))
        frac = len(hsel) / H
        cpu_model = None
        try:
            with open("/proc/cpuinfo") as fh:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh
                                  if ln.startswith("model name")), None)
        except OSError:
            pass
        cpu = {"value": round(T * frac / wall, 1), "unit": "tokens/s", "cores": threads,
               "cpu_model": cpu_model, "kind": "oracle",
               "sample": f"{w.name}: all {T} tokens x {len(hsel)} of {H} heads, run {len(walls)}x "
                         f"({cpu_s:.1f} CPU-s in total); median {wall:.3f} s wall per run"
                         + ("" if frac == 1 else "; tokens/s scaled to all heads")}
        og = wl.bf16_tensor_to_f32(o_check[:, hsel]).astype(np.float64)
        fg = f_check[:, hsel].cpu().numpy().astype(np.float64)
        parity = {"heads_checked": len(hsel),
                  "o_maxabs": oracle.max_abs_err(og, o_or), "o_relF": oracle.rel_fro_err(og, o_or),
                  "final_maxabs": oracle.max_abs_err(fg, f_or),
                  "final_relF": oracle.rel_fro_err(fg, f_or)}
        parity = {k: (float(f"{v:.3e}") if isinstance(v, float) else v) for k, v in parity.items()}

    out = {
        "metric": METRIC, "value": round(T / step_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "N": N, "H": H, "K": 128, "V": 128, "BT": 64,
                   "SB": 16, "chunks": nc, "initial_state": w.initial_state is not None,
                   "input_copies_rotated": R,
                   "settle": {"seconds": args.settle_seconds, "steps": settle_steps}},
        "roofline": roofline, "path": path, "cpu_baseline": cpu, "parity_vs_oracle": parity,
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
