#!/usr/bin/env python3
"""Benchmark: exact softmax attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_16k_causal]

One step = one forward over the whole batch of the workload (all of the hot path runs in
one kernel launch). The default workload is the long-context causal one, B=1 H=16 N=16384
d=128 (the paper's Figure 5d point at 16k tokens). Inputs are generated once,
copied to HBM, and stay resident; the timed region covers K launches bracketed by
synchronisations, timed with HIP events recorded on the stream the kernels are launched on
(torch's current stream, which the binding passes to the C ABI).

Metric: attention forward TFLOP/s with FLOPs = 4*B*H*N^2*d, halved for causal (the paper's
accounting; paper-graph-ui summary, "5. Experimental Analysis", Metrics), and the fraction
of MI355X's dense bf16 MFMA peak.

Prints ONE JSON line. ``roofline.traffic`` comes from rocprofv3 FETCH_SIZE/WRITE_SIZE
counter runs ingested with ``--ingest-counters`` (stored under profiles/ together with the
hash of the kernel source they were taken on); it is null when the source has changed
since. ``cpu_baseline`` times the CPU fp64 oracle on a bounded sample of the same workload.
``launch_ms`` repeats the K steps with one event pair each (median, min, max of single
launches); ``gpu_clock`` is the shader clock and board power sampled with amd-smi during
about a second of further untimed steps (null where amd-smi is absent; ``--no-clock`` skips
it). Neither changes ``value``.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU (published 2.5 PF)
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_MHZ = 2400.0   # the shader clock the published peak is quoted at
A100_FIG5D_16K_TFLOPS = 197.0   # the pages' FA2 forward, causal, d=128, 16k (A100; context only)
KERNEL_SRCS = [os.path.join(ROOT, "exact_softmax_attention_amd", "csrc", name) for name in ("fa2_fwd.hip", "fa2_dev.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa2_fwd_long16k_traffic.json")
WORKLOAD_NAMES = ("single_head_256", "batch8_2k_d128", "batch8_2k_d64_causal", "long_16k_causal", "varlen16_causal")
COPY_BYTES = 1 << 30   # the calibration copy kernel moves 1 GiB in and 1 GiB out
WARMUP_SECONDS = 0.5   # default warmup: untimed work before the timed steps, in seconds
CLOCK_SECONDS = 1.0    # untimed steps after the timed ones while amd-smi samples the shader clock


def kernel_source_hash() -> str:
    """Hash of the forward kernel's code (the kernel file and the device helpers it includes),
    with `//` comments, trailing blanks and empty lines left out, so that an edit to a comment
    does not mark the stored counters as stale. The sources use no `/* */` comments and no
    `//` inside string literals."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def algorithmic_bytes(w, lengths=None, kv_heads=None) -> int:
    """Q, K, V read once and O written once (bf16), LSE written once (fp32); K and V have
    kv_heads heads (grouped-query attention), H by default."""
    hk = w.H if kv_heads is None else kv_heads
    if w.varlen:
        T = sum(lengths)
        return 4 * (w.H + hk) * T * w.d + 4 * w.H * T
    return 4 * w.B * (w.H + hk) * w.N * w.d + 4 * w.B * w.H * w.N


def bwd_algorithmic_bytes(w, kv_heads=None, lengths=None) -> int:
    """Backward: read Q, K, V, O, dO and LSE once, write dQ, dK, dV once (bf16); D is
    written and read once (fp32)."""
    hk = w.H if kv_heads is None else kv_heads
    tokens = sum(lengths) if w.varlen else w.B * w.N
    rows_q, rows_kv = w.H * tokens, hk * tokens
    return 2 * w.d * (4 * rows_q + 4 * rows_kv) + 4 * rows_q + 8 * rows_q


def load_traffic():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t


def host_cpu_info() -> dict:
    """CPU model, physical cores and logical CPUs of this host (lscpu), and the CPUs this
    process may run on."""
    import subprocess
    info = {"logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return info
    fields = {}
    for line in out.splitlines():
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    info["model"] = fields.get("Model name")
    try:
        info["physical_cores"] = int(fields["Core(s) per socket"]) * int(fields["Socket(s)"])
    except (KeyError, ValueError):
        pass
    return info


def cpu_baseline(w, q, k, v, heads: int):
    """Time the fp64 oracle on `heads` heads of batch 0 (all rows)."""
    import numpy as np
    from oracle import attention_head
    from synthetic import metric_flops
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:
        threads = 1
    t0 = time.perf_counter()
    for h in range(heads):
        attention_head(q[0, h].double().numpy(), k[0, h].double().numpy(), v[0, h].double().numpy(),
                       w.causal, w.scale)
    dt = time.perf_counter() - t0
    f = metric_flops(1, heads, w.N, w.d, w.causal)
    return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} (batch, head) pairs, all {w.N} rows, fp64 numpy "
                      f"({dt:.2f} s; cores = the BLAS threads it ran on)",
            "seconds": dt, "host": host_cpu_info()}


def parse_amdsmi_metric(text: str):
    """Shader clocks (MHz, one per XCD) and socket power (W) of the first GPU in the JSON
    printed by ``amd-smi metric -p -c --json``; (None, None) for what is missing."""
    try:
        data = json.loads(text)
    except (ValueError, TypeError):
        return None, None
    if isinstance(data, dict):
        data = data.get("gpu_data", [data])
    if not isinstance(data, list) or not data or not isinstance(data[0], dict):
        return None, None
    gpu = data[0]
    clocks = []
    for name, entry in sorted((gpu.get("clock") or {}).items()):
        clk = entry.get("clk") if isinstance(entry, dict) and name.startswith("gfx") else None
        if isinstance(clk, dict) and isinstance(clk.get("value"), (int, float)):
            clocks.append(float(clk["value"]))
    power = ((gpu.get("power") or {}).get("socket_power") or {}).get("value")
    return (clocks or None), (float(power) if isinstance(power, (int, float)) else None)


def sample_gpu_clock(step, seconds: float = CLOCK_SECONDS):
    """Run ``step`` back to back for about ``seconds`` while amd-smi samples the shader clocks
    and the board power. Returns medians over the samples, or None without amd-smi."""
    import shutil
    import subprocess
    import threading

    import torch

    smi = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if smi is None:
        return None
    samples, done = [], threading.Event()

    def poll():
        while not done.is_set():
            try:
                r = subprocess.run([smi, "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            clocks, power = parse_amdsmi_metric(r.stdout) if r.returncode == 0 else (None, None)
            if clocks:
                samples.append((sum(clocks) / len(clocks), min(clocks), max(clocks), power))

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds or (not samples and time.perf_counter() - t0 < 4 * seconds):
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    done.set()
    th.join(timeout=15)
    if not samples:
        return None
    med = lambda xs: sorted(xs)[len(xs) // 2]
    powers = [x[3] for x in samples if x[3] is not None]
    return {"gfx_mhz_median": med([x[0] for x in samples]), "gfx_mhz_min": min(x[1] for x in samples),
            "gfx_mhz_max": max(x[2] for x in samples),
            "socket_power_w_median": med(powers) if powers else None,
            "samples": len(samples), "source": "amd-smi metric -p -c (mean over XCDs per sample)"}


def default_warmup(seconds_per_step: float) -> int:
    """Untimed steps for about WARMUP_SECONDS of work: 5 probe steps, then at least 5 and at
    most 20000 more."""
    return 5 + max(5, min(20000, math.ceil(WARMUP_SECONDS / max(seconds_per_step, 1e-6))))


def run(args):
    import torch

    import exact_softmax_attention_amd as fa2
    from synthetic import WORKLOADS, metric_flops, varlen_metric_flops, workload_inputs

    w = WORKLOADS[args.workload]
    if args.head_dim:
        import dataclasses
        if w.varlen:
            raise SystemExit("--head-dim applies to fixed-length workloads")
        w = dataclasses.replace(w, d=args.head_dim,
                                description=w.description.replace(f"d={w.d}", f"d={args.head_dim}"))
    dev = torch.device("cuda:0")
    lengths = None
    # The default kernel is timed through the C ABI's plain entry points (fa2_fwd,
    # fa2_fwd_varlen); another variant through the *_variant calls.
    entry_variant = None if args.variant == 0 else args.variant
    if w.varlen:
        if args.kv_heads:
            from synthetic import make_varlen
            if w.H % args.kv_heads:
                raise SystemExit(f"--kv-heads {args.kv_heads} must divide H={w.H}")
            q, k, v, cu, lengths = make_varlen(w.H, w.d, w.seed, num_seqs=w.num_seqs, min_len=w.min_len,
                                               max_len=w.max_len, k_scale=w.k_scale, H_kv=args.kv_heads)
        else:
            q, k, v, cu, lengths = workload_inputs(w)
        qd, kd, vd, cud = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:2], dtype=torch.float32, device=dev)
        maxlen = max(lengths)
        flops = varlen_metric_flops(lengths, w.H, w.d, w.causal)

        varlen_fwd = fa2.fwd_varlen_gqa if args.kv_heads else fa2.fwd_varlen

        def step():
            varlen_fwd(qd, kd, vd, cud, maxlen, causal=w.causal, scale=w.scale, out=o, lse=lse,
                       variant=entry_variant)
    elif args.kv_heads:
        from synthetic import make_qkv
        if w.H % args.kv_heads:
            raise SystemExit(f"--kv-heads {args.kv_heads} must divide H={w.H}")
        q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.seed, w.k_scale, H_kv=args.kv_heads)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        flops = metric_flops(w.B, w.H, w.N, w.d, w.causal)

        def step():
            fa2.fwd_gqa(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, variant=args.variant)
    else:
        q, k, v = workload_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        flops = metric_flops(w.B, w.H, w.N, w.d, w.causal)

        def step():
            fa2.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, variant=entry_variant)

    merge_info = None
    if args.split_kv:
        if w.varlen or args.bwd or args.fwd_bwd or args.kv_heads:
            raise SystemExit("--split-kv runs the forward of a fixed-length MHA workload")
        S, N = args.split_kv, w.N
        nq = args.q_rows or N
        if N % S or not (0 < nq <= N):
            raise SystemExit(f"--split-kv {S} must divide N={N}; 0 < --q-rows <= N")
        step_k = N // S
        qq = qd[:, :, N - nq:].contiguous()
        o_parts = torch.empty((S,) + tuple(qq.shape), dtype=torch.bfloat16, device=dev)
        l_parts = torch.empty((S,) + tuple(qq.shape[:3]), dtype=torch.float32, device=dev)
        o = torch.empty_like(qq)
        lse = torch.empty(qq.shape[:3], dtype=torch.float32, device=dev)
        if nq < N:    # exact count of allowed (query, key) pairs, bottom-right causal
            pairs = nq * (N - nq) + nq * (nq + 1) // 2 if w.causal else nq * N
            flops = 4.0 * w.d * w.B * w.H * pairs

        def step():   # all pieces in one launch, then the merge
            fa2.fwd_splitkv(qq, kd, vd, S, causal=w.causal, diag=N - nq, scale=w.scale, out=o, lse=lse,
                            o_parts=o_parts, lse_parts=l_parts, variant=args.variant)

        def one_pass():
            fa2.fwd_chunk(qq, kd, vd, causal=w.causal, diag=N - nq, scale=w.scale, out=o, lse=lse,
                          variant=args.variant)

        def merge_only():
            fa2.lse_merge(o_parts, l_parts, out=o, lse=lse)

        rows = qq.numel() // w.d
        merge_info = {"parts": S, "q_rows": nq, "rows": rows,
                      "merge_bytes": S * rows * (2 * w.d + 4) + rows * (2 * w.d + 4),
                      "fns": (one_pass, merge_only)}

    if args.bwd or args.fwd_bwd:
        gen = torch.Generator(device="cpu").manual_seed(1000 + w.seed)
        dod = torch.randn(qd.shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).to(dev)
        if w.varlen:
            fwd_step = lambda: varlen_fwd(qd, kd, vd, cud, maxlen, causal=w.causal, scale=w.scale, out=o,
                                          lse=lse, variant=entry_variant)
        elif kd.shape[1] == qd.shape[1]:
            fwd_step = lambda: fa2.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse,
                                       variant=entry_variant)
        else:
            fwd_step = lambda: fa2.fwd_gqa(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse,
                                           variant=args.variant)
        fwd_step()
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        delta = torch.empty_like(lse)
        fwd_flops = flops
        flops = 2.5 * flops   # five matrix products against the forward's two

        if w.varlen:
            def step():
                fa2.bwd_varlen(qd, kd, vd, o, lse, dod, cud, maxlen, causal=w.causal, scale=w.scale, dq=dq, dk=dk,
                               dv=dv, delta=delta)
        else:
            def step():
                fa2.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                        delta=delta)

        if args.fwd_bwd:      # one training step of the attention: the forward, then the backward
            flops += fwd_flops
            bwd_step = step

            def step():
                fwd_step()
                bwd_step()

    if args.calib_copy:   # a plain copy kernel of known size, for counter calibration
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream(dev)
    # Clock settle: untimed launches for about args.settle seconds before the warm-up steps,
    # so that a short warm-up count (e.g. --warmup 5) does not time the shader clock's ramp
    # from idle. Reported as settle_launches; the warm-up steps and the timed steps follow
    # unchanged.
    settle_launches = 0
    if args.settle > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle:
            for _ in range(4):
                step()
            settle_launches += 4
            torch.cuda.synchronize()
    if args.warmup is None:
        # Untimed steps until about WARMUP_SECONDS of work has run, so that the shader clock
        # has settled (a short kernel timed from a cold start reads up to 20% slow). The
        # probe steps count towards the reported warmup.
        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(4):
            step()
        torch.cuda.synchronize()
        args.warmup = default_warmup((time.perf_counter() - t0) / 4)
        for _ in range(args.warmup - 5):
            step()
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # The K steps captured once in a HIP graph (every entry point only enqueues kernel
        # launches), so the timed region is one graph launch: no per-step host overhead.
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        graph.replay()                    # one untimed replay
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12

    # The same steps once more, each between its own pair of events on the launch stream:
    # the spread of single launches (median, min, max), reported beside the mean above.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    single = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    launch_ms = {"median": round(single[len(single) // 2], 5), "min": round(single[0], 5),
                 "max": round(single[-1], 5), "n": len(single)} if single else None
    gpu_clock = sample_gpu_clock(step) if args.clock else None
    if gpu_clock:
        # the dense peak scaled to the sampled clock (the published peak assumes 2.4 GHz)
        at_clock = PEAK_BF16_TFLOPS * gpu_clock["gfx_mhz_median"] / PEAK_CLOCK_MHZ
        gpu_clock.update(peak_at_clock_tflops=round(at_clock, 1), frac_at_clock=round(tflops / at_clock, 4))

    def time_fn(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    split_report = None
    if merge_info is not None:
        one_pass, merge_only = merge_info.pop("fns")
        one_ms = time_fn(one_pass, args.steps)
        merge_ms = time_fn(merge_only, max(args.steps, 20))
        gbs = merge_info["merge_bytes"] / (merge_ms * 1e-3) / 1e9
        split_report = dict(merge_info, one_pass_ms=round(one_ms, 5),
                            one_pass_tflops=round(flops / (one_ms * 1e-3) / 1e12, 2),
                            merge_ms=round(merge_ms, 5),
                            merge_roofline={"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)})
        # With few query rows (decoding) the step is bound by streaming K and V once: report
        # that rate for the whole step (pieces and merge).
        kv_bytes = 2 * w.B * w.H * w.N * w.d * 2
        kv_gbs = kv_bytes / (ms * 1e-3) / 1e9
        split_report.update(kv_bytes=kv_bytes,
                            step_kv_roofline={"bound": "hbm", "achieved": round(kv_gbs, 1), "peak": PEAK_HBM_GBS,
                                              "unit": "GB/s", "frac": round(kv_gbs / PEAK_HBM_GBS, 4)})

    traffic = None
    t = (load_traffic() if (w.name == "long_16k_causal" and args.variant == 0
                            and not (args.kv_heads or args.bwd or args.fwd_bwd or args.split_kv or args.head_dim))
         else None)
    if t is not None:
        traffic = t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]

    # fa2_fwd_varlen picks its own variant; report the one it runs.
    variant = fa2.variant_name(w.d, fa2.varlen_default_variant(w.d) if (w.varlen and args.variant == 0)
                               else args.variant)
    config = {"workload": f"{w.name}: {w.description}", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
              "causal": w.causal, "kernel_variant": variant}
    if args.graph:
        config["timing"] = f"{args.steps} steps captured in one HIP graph, one replay timed"
    if w.varlen:
        config.update({"lengths": lengths, "total_tokens": sum(lengths)})
    if args.kv_heads:
        config.update({"workload": f"{w.name} with grouped-query K/V: {w.description}, "
                                   f"{args.kv_heads} key/value heads", "H_kv": args.kv_heads})
    if args.bwd:
        config.update({"workload": f"backward of {config['workload']}", "kernel_variant": "bwd_dq+bwd_dkdv"})
    if args.fwd_bwd:
        config.update({"workload": f"forward then backward of {config['workload']}",
                       "kernel_variant": f"{variant}+bwd_dq+bwd_dkdv"})
    if split_report is not None:
        config.update({"workload": f"split-KV forward ({split_report['parts']} key pieces in one launch + LSE merge), last "
                                   f"{split_report['q_rows']} queries of {config['workload']}",
                       "split_kv": split_report})
    out = {
        "metric": ("attention bwd TFLOP/s (2.5 x 4*B*H*N^2*d, causal halved) + % of bf16 MFMA peak" if args.bwd
                   else "attention fwd+bwd TFLOP/s (3.5 x 4*B*H*N^2*d, causal halved) + % of bf16 MFMA peak"
                   if args.fwd_bwd
                   else "attention fwd TFLOP/s (4*B*H*N^2*d, causal halved) + % of bf16 MFMA peak"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "settle_launches": settle_launches,
        "higher_is_better": True,
        "scaling": "weak",
        # The pages print this workload's figure only for another machine (A100): context,
        # reported beside the line, not as the baseline ratio.
        "vs_baseline": None,
        "pages_a100": ({"tflops": A100_FIG5D_16K_TFLOPS, "ratio": round(tflops / A100_FIG5D_16K_TFLOPS, 3),
                        "basis": "the pages' FA2 forward figure for this workload (causal, d=128, 16k tokens, "
                                 "Figure 5d), measured on A100; another machine's number, context only"}
                       if w.name == "long_16k_causal"
                       and not (args.kv_heads or args.bwd or args.fwd_bwd or args.split_kv or args.head_dim)
                       else None),
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_bytes": (bwd_algorithmic_bytes(w, args.kv_heads or None, lengths) if args.bwd
                                  else algorithmic_bytes(w, lengths, args.kv_heads or None)
                                  + bwd_algorithmic_bytes(w, args.kv_heads or None, lengths) if args.fwd_bwd
                                  else algorithmic_bytes(w, lengths, args.kv_heads or None)),
            "flops_per_launch": flops,
            "kernel_ms": round(ms, 5),
        },
        "launch_ms": launch_ms,
        "gpu_clock": gpu_clock,
    }
    if args.cpu_baseline_heads > 0:
        out["cpu_baseline"] = (cpu_baseline(w, q, k, v, min(args.cpu_baseline_heads, w.H))
                               if not (w.varlen or args.kv_heads or args.bwd or args.fwd_bwd or args.split_kv
                                       or args.head_dim)
                               else None)
    print(json.dumps(out), flush=True)


def ingest_counters(fetch_csv: str, write_csv: str, steps: int):
    """Turn two rocprofv3 --pmc counter_collection CSVs (FETCH_SIZE, WRITE_SIZE) into the
    per-launch HBM traffic of the attention kernel, scaled by the calibration copy kernel."""
    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                vals.setdefault(name, []).append(float(row["Counter_Value"]))
        return vals

    out = {"kernel_source_sha256": kernel_source_hash()}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        attn = [v for n, vs in vals.items() if "fa2_fwd_kernel" in n for v in vs]
        # the calibration copy: the largest other kernel; it moves COPY_BYTES each way, and a
        # counter that sees it must report at least a quarter of that
        others = [max(vs) for n, vs in vals.items() if "fa2_fwd_kernel" not in n]
        copy = max(others) if others else 0.0
        if not attn or copy < COPY_BYTES / 1024 / 4:
            raise SystemExit(f"{path}: need both the attention kernel and the calibration copy")
        factor = (COPY_BYTES / 1024) / copy               # counter reads KiB
        per_launch = sorted(attn)[len(attn) // 2] * 1024 * factor
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        out[f"{key}_bytes_per_launch"] = per_launch
        out[f"{key}_copy_factor"] = factor
        out[f"{key}_raw_kib_median"] = sorted(attn)[len(attn) // 2]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help=f"untimed warmup steps (default: as many as take about {WARMUP_SECONDS} s, at least 10)")
    ap.add_argument("--workload", default="long_16k_causal", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward (dQ, dK, dV from dO, O, LSE) instead of the forward")
    ap.add_argument("--graph", action="store_true",
                    help="time the K steps as one captured HIP graph (no per-launch host overhead)")
    ap.add_argument("--fwd-bwd", action="store_true",
                    help="time the forward followed by the backward (one attention training step)")
    ap.add_argument("--split-kv", type=int, default=0,
                    help="split the keys into this many pieces in one launch and merge them (fa2_fwd_splitkv)")
    ap.add_argument("--q-rows", type=int, default=0,
                    help="with --split-kv: only the last Q_ROWS queries (decode / chunked prefill shape)")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="override the workload's head dimension (64, 128 or 256)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="grouped-query attention: K/V with this many heads (must divide H; 0: H)")
    ap.add_argument("--cpu-baseline-heads", type=int, default=16,
                    help="(batch, head) pairs of batch 0 the CPU oracle is timed on, all rows (0: skip; "
                         "16 = every head of the long-context workload, about 30 s on a 16-core host)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="untimed seconds of launches before the warm-up steps (clock settle; 0: none)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB copy kernel (counter calibration for --ingest-counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--no-clock", dest="clock", action="store_false",
                    help=f"skip the shader-clock sample (amd-smi, about {CLOCK_SECONDS} s of extra untimed steps)")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, steps=args.steps)
        return
    if args.bwd and args.fwd_bwd:
        ap.error("--bwd and --fwd-bwd are exclusive")
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards across GPUs by (batch, head) with no communication; only the "
              "one-GPU share is implemented).", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
