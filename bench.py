"""Benchmark of the causal FoX attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--no-cpu-baseline] [--only]

A step is one call of the library entry point on one batch of synthetic,
seeded, device-resident input:
  * fox_attn_fwd (gate scan fused in; one kernel) for the forward workloads,
  * fox_attn_decode (split + combine kernels) for the decode workload.
The headline workload is the largest single-GPU forward configuration, bf16
B=1 H=32 N=16384 d=128 (the metric names no configuration); the JSON line also
carries the other forward workloads, the backward and the decode workload (the
metric quotes prefill TFLOP/s and decode GB/s), each with its roofline, unless
--only is given.

Timing: W untimed warm-up steps, then K back-to-back steps between two HIP events
on the stream the library launches on (torch's current stream), bracketed by
synchronisation.  A forward step is exactly one kernel launch, so the region time
over K is also that kernel's average launch duration, which the roofline object
uses (per-launch event pairs would add their own overhead to a 25 us kernel); a
decode step is its split kernel plus the small combine kernel.

Algorithmic work (what the method must do, not what the kernel happens to do):
  forward: 4*d flop per causal pair, n(n+1)/2 pairs per (batch, head);
  decode : bytes = K and V caches + cached prefix sums (L-1 slots) + q + log f_new
           read, O + lse + c_{L-1} written.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 matrix / vector
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "causal FoX attn fwd TFLOP/s (% bf16 MFMA peak); decode GB/s (% HBM peak)"


def fwd_flops(cfg) -> float:
    return 4.0 * cfg.d * cfg.N * (cfg.N + 1) / 2 * cfg.B * cfg.H


def decode_bytes(cfg, lens=None) -> dict:
    """Algorithmic bytes of one decode call; with per-sequence lengths, only the slots in use."""
    eb = 2 if cfg.dtype == "bf16" else 4
    slots = cfg.S * cfg.L if lens is None else int(sum(int(x) for x in lens))
    sh = cfg.S * cfg.H
    kv = 2 * cfg.H * slots * cfg.d * eb
    rd = kv + cfg.H * (slots - cfg.S) * 4 + sh * cfg.d * eb + sh * 4
    wr = sh * cfg.d * eb + sh * 4 + sh * 4
    return {"total": rd + wr, "read": rd, "kv": kv, "write": wr}


# HBM-side traffic of the dominant kernel comes from rocprofv3 counter runs (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a plain device
# copy of known size.  The summaries live in profiles/*_traffic.txt with a digest of the kernel
# sources they were taken on; a summary of older sources is not used (traffic reported as null).
KERNEL_SOURCES = {"fwd": ["fox_fwd.hip", "fox_fwd_gates.h", "fox_device.h"], "decode": ["fox_decode.hip", "fox_device.h"],
                  "bwd": ["fox_bwd.hip", "fox_scan.hip", "fox_device.h"]}
COPY_CAL_BYTES = 1 << 30
DECODE_KERNEL = "decode_split_kernel<bf16,128> + decode_combine_kernel<bf16,128>"
BWD_KERNEL = "fox_attn_bwd<{d},causal>: bwd_rows (gate rows + D) + bwd_kv + bwd_dq + suffix scan"
BWD_STAGED_KERNEL = ("fox_attn_bwd_staged<{d}>: bwd_rows (gate rows + D) + bwd_kv (dS staged) + bwd_dq_staged "
                     "+ suffix scan")


def kernel_source_digest(kind: str) -> str:
    """Digest of the sources a kernel kind is built from, with their per-source compiler flags."""
    from forget_gated_causal_amd.build import SOURCE_FLAGS
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "forget_gated_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
        if SOURCE_FLAGS.get(f):
            h.update(" ".join(SOURCE_FLAGS[f]).encode())
    return h.hexdigest()[:16]


def _read_summary(path):
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def stored_traffic(tag: str, kernel: str, kind: str):
    """Bytes per launch of `kernel` on workload `tag` from a committed counter summary, or None."""
    digest = kernel_source_digest(kind)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt"))):
        kv = _read_summary(path)
        if kv.get("workload") == tag and kv.get("kernel") == kernel and kv.get("source_digest") == digest:
            return float(kv["traffic_bytes_per_launch"])
    return None


def _counter_per_dispatch(path, counter, name_part):
    """Mean value of `counter` per dispatch of each kernel whose name contains name_part (or one
    of its "|"-separated parts), summed over those kernels (one call of an entry point that
    launches several kernels); and the number of dispatches of the first of them."""
    tot, ids = {}, {}
    parts = name_part.split("|")
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter and any(p in r["Kernel_Name"] for p in parts):
                k = r["Kernel_Name"]
                tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
                ids.setdefault(k, set()).add(r["Dispatch_Id"])
    if not tot:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {name_part!r}")
    return sum(tot[k] / len(ids[k]) for k in tot), min(len(v) for v in ids.values())


def write_traffic_summary(args):
    """Combine four rocprofv3 --pmc CSVs (kernel FETCH/WRITE, copy FETCH/WRITE) into a summary."""
    fetch, nf = _counter_per_dispatch(args.fetch_csv, "FETCH_SIZE", args.kernel_match)
    write, nw = _counter_per_dispatch(args.write_csv, "WRITE_SIZE", args.kernel_match)
    cf, _ = _counter_per_dispatch(args.copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_per_dispatch(args.copy_write_csv, "WRITE_SIZE", "copyBuffer")
    f_fac, w_fac = COPY_CAL_BYTES / (cf * 1024), COPY_CAL_BYTES / (cw * 1024)
    rd, wr = fetch * 1024 * f_fac, write * 1024 * w_fac
    lines = [
        f"# rocprofv3 counter summary: HBM-side traffic per launch of {args.kernel} on workload {args.workload}",
        "# commands (one counter per run; <out> is the output directory):",
        f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch -o p -- python3 bench.py --workload {args.workload} "
        f"--only --no-cpu-baseline --steps 4 --warmup 2{' --backward' if args.kind == 'bwd' else ''}{' --staged' if getattr(args, 'staged', False) else ''}",
        f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write -o p -- python3 bench.py --workload {args.workload} "
        f"--only --no-cpu-baseline --steps 4 --warmup 2{' --backward' if args.kind == 'bwd' else ''}{' --staged' if getattr(args, 'staged', False) else ''}",
        "#   rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/copy_fetch -o p -- python3 bench.py --copy-calibration",
        "#   rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/copy_write -o p -- python3 bench.py --copy-calibration",
        "#   python3 bench.py --traffic-summary ... (this file)",
        "# calibration: a device copy of 1 GiB reads as FETCH_SIZE "
        f"{cf:.1f} KiB and WRITE_SIZE {cw:.1f} KiB, so the factors are {f_fac:.4f} (read) and {w_fac:.4f} (write)",
        f"workload: {args.workload}",
        f"kernel: {args.kernel}",
        f"source_digest: {kernel_source_digest(args.kind)}",
        f"dispatches: {nf} (FETCH_SIZE run), {nw} (WRITE_SIZE run)",
        f"fetch_kib_per_dispatch: {fetch:.1f}",
        f"write_kib_per_dispatch: {write:.1f}",
        f"read_bytes_per_launch: {rd:.0f}",
        f"write_bytes_per_launch: {wr:.0f}",
        f"traffic_bytes_per_launch: {rd + wr:.0f}",
    ]
    if args.alg_bytes:
        lines.append(f"algorithmic_bytes_per_launch: {args.alg_bytes:.0f}")
        lines.append(f"traffic_over_algorithmic: {(rd + wr) / args.alg_bytes:.3f}")
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_trace_summary(args):
    """A rocprofv3 --kernel-trace --stats table (kernel_stats.csv) plus the bench lines that the same
    run printed, as a short text summary."""
    with open(args.stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    bench_lines = []
    if args.bench_log:
        with open(args.bench_log) as fh:
            bench_lines = [l.rstrip() for l in fh if l.startswith("# fox_")]
    lines = [f"# rocprofv3 kernel-trace summary: {args.title}",
             "# command (<out> is the output directory):",
             f"#   cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d <out> -o t -- python3 <repo>/bench.py {args.bench_args}",
             f"#   python3 bench.py --trace-summary ... (this file)"]
    lines += [f"# {n}" for n in (args.note or [])]
    if bench_lines:
        lines.append("# bench.py's own lines from the same run (HIP events around the timed calls):")
        lines += ["#   " + b[:400] for b in bench_lines]
    lines += ["", f"{'kernel':100s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_ms':>9s}"]
    for r in rows:
        lines.append(f"{r['Name'][:100]:100s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                     f"{float(r['TotalDurationNs']) / 1e6:9.3f}")
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _demangle(name: str) -> str:
    """Short readable name of one of this library's kernels from its mangled symbol: the name and its
    integer / bool template arguments (e.g. fwd_bf16_pipe_kernel<128,8,1,0,1,0>); other names as given."""
    m = re.match(r"_ZN3fox12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    pos = m.end() + int(m.group(1))
    ident = name[m.end():pos]
    vals = []
    if name[pos:pos + 1] == "I":
        pos += 1
        arg = re.compile(r"L[ib](-?\d+)E")
        while (a := arg.match(name, pos)) is not None:
            vals.append(a.group(1))
            pos = a.end()
    return f"{ident}<{','.join(vals)}>" if vals else ident


# algorithmic flop per causal pair of each MFMA kernel (the backward's parts count their own share)
MFMA_KERNEL_FLOP_PER_PAIR_D = {"fwd_bf16_pipe_kernel": 4, "bwd_kv_kernel": 8, "bwd_dq_kernel": 6,
                               "bwd_dq_staged_kernel": 2}


def write_mfma_summary(args):
    """MFMA use per kernel from rocprofv3 --pmc runs of SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU_MFMA_MOPS_BF16 and GRBM_GUI_ACTIVE; --pmc-csv takes workload:kind:path triples."""
    import fox_inputs as fi
    lines = ["# rocprofv3 counter summary: MFMA use per kernel",
             "# commands (one run per workload; <out> is the output directory):",
             "#   cd /tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE -f csv \\",
             "#     -d <out>/<w>_<kind> -o p -- python3 <repo>/bench.py --workload <w> --only --no-cpu-baseline --steps 4 "
             "--warmup 2 [--backward [--staged]]",
             "#   python3 bench.py --mfma-summary ... (this file)",
             "# per dispatch (mean over every dispatch of the kernel in the run, warm-up included):",
             "#   mfma_flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (bf16 MFMA flops executed, masked diagonal halves included)",
             "#   mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs * GRBM_GUI_ACTIVE / 8); GRBM_GUI_ACTIVE is summed over",
             "#               the 8 XCDs; the busy counter reads 32 cycles per 32x32x16 bf16 MFMA",
             "#   alg_flop  = 4 d (forward), 8 d (backward key side), 6 d (backward query side, which recomputes S and",
             "#               dP), 2 d (the staged-dS backward's dQ kernel) per causal pair",
             "",
             f"{'workload':10s} {'kernel':44s} {'disp':>5s} {'dur_us':>9s} {'mfma_flop':>11s} {'alg_flop':>11s} "
             f"{'exec/alg':>8s} {'mfma_util':>9s}"]
    for spec in args.pmc_csv:
        tag, kind, path = spec.split(":", 2)
        kind = "bwd" if kind == "bwd_staged" else kind
        cfg = fi.FWD[tag]
        pairs = cfg.B * cfg.H * cfg.N * (cfg.N + 1) / 2
        per = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                k = r["Kernel_Name"]
                d = per.setdefault(k, {"ids": set(), "dur": {}, "c": {}})
                d["ids"].add(r["Dispatch_Id"])
                d["dur"][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for k, d in per.items():
            if not k.startswith("void fox::") and "fox" not in k:
                continue
            n = len(d["ids"])
            mops = d["c"].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) / n
            busy = d["c"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n
            act = d["c"].get("GRBM_GUI_ACTIVE", 0.0) / n / 8
            dur = sum(d["dur"].values()) / n / 1e3
            short = _demangle(k).replace("fox::(anonymous namespace)::", "").replace("void ", "")
            short = short.split("(")[0].replace(" ", "")
            if kind == "bwd" and short.startswith("fwd_"):
                continue  # the forward that makes the backward's inputs
            alg = next((m * cfg.d * pairs for nm, m in MFMA_KERNEL_FLOP_PER_PAIR_D.items() if nm in short), 0.0)
            util = busy / (1024 * act) if act else 0.0
            ratio = f"{mops * 512 / alg:8.3f}" if alg else f"{'-':>8s}"
            lines.append(f"{tag:10s} {short[:44]:44s} {n:5d} {dur:9.2f} {mops * 512:11.4e} {alg:11.4e} {ratio} "
                         f"{100 * util:8.1f}%")
    lines += [f"# {n}" for n in (args.note or [])]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, three times (counter calibration)."""
    import torch
    x = torch.empty(COPY_CAL_BYTES // 4, device="cuda", dtype=torch.float32).fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {COPY_CAL_BYTES} bytes x 3", flush=True)


def fwd_min_bytes(cfg) -> float:
    """Bytes the forward must move: q, k, v, log f read; o, lse, c written."""
    eb = 2 if cfg.dtype == "bf16" else 4
    rows = cfg.B * cfg.H * cfg.N
    return rows * cfg.d * eb * 4 + rows * 4 * 3


def _warm(torch, fn, warmup, min_s=0.05):
    """W untimed calls, then more until at least min_s of wall time has passed on the device
    (clocks ramp up under load; a short workload measured after an idle host phase would
    otherwise be timed partly at a lower clock)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


USE_GRAPH = False  # bench.py --graph: time a captured graph of the calls instead


def _events_time(torch, fn, k):
    """Time (ms) of k back-to-back calls between two events on the launch stream.

    With --graph the k calls are captured once into a HIP graph (the entry points only launch
    kernels on the caller's stream) and the graph is replayed between the events, after one
    untimed replay: the host's per-call cost (a profiler's interception, say) then cannot leave
    the device idle between launches, at the price of the graph's own gap between nodes (about
    1 us per call measured on c2).  By default the calls are launched directly."""
    st = torch.cuda.current_stream()
    if USE_GRAPH:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(k):
                fn()
        g.replay()
        run = g.replay
    else:
        def run():
            for _ in range(k):
                fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    run()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def fwd_kernel_name(torch, cfg, causal: bool = True) -> str:
    """The kernel fox_attn_fwd launches for this shape (same rule as the library's dispatch)."""
    if cfg.dtype != "bf16":
        return f"fwd_f32_kernel<{cfg.d}>"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bh = cfg.B * cfg.H
    if cfg.d >= 64 and bh * ((cfg.N + 255) // 256) >= 2 * cus:
        return f"fwd_bf16_pipe_kernel<{cfg.d},8,1>"
    blocks128 = bh * ((cfg.N + 127) // 128)
    if cfg.d <= 64 and blocks128 < 2 * cus and (causal or blocks128 <= cus):
        return f"fwd_bf16_pipe_kernel<{cfg.d},4,2>"
    return f"fwd_bf16_pipe_kernel<{cfg.d},4,1>"


def bench_fwd(torch, fox, fi, tag, steps, warmup, mode="causal"):
    """mode: "causal" (fox_attn_fwd), "unmasked" (fox_attn_fwd_noncausal, 4*d flop for every
    (query, key) pair), "pruned" (fox_attn_fwd_pruned, timed whole with its key-norm and
    prefix-sum kernels; its rate is the causal work over that time, an effective rate) or
    "token" (fox_attn_fwd_ex on [B,N,H,d] tensors, causal)."""
    cfg = fi.FWD[tag]
    inp = fi.fwd_inputs(cfg)
    dev = "cuda"
    q, k, v, logf = (inp[n].to(dev) for n in ("q", "k", "v", "logf"))
    o = torch.empty_like(q)
    lse = torch.empty_like(logf)
    c = torch.empty_like(logf)
    if mode == "unmasked":
        fn = lambda: fox.attn_fwd_noncausal(q, k, v, logf, scale=inp["scale"], out=o, lse=lse, c=c)  # noqa: E731
    elif mode == "pruned":
        ws = torch.empty(max(16, fox.attn_fwd_pruned_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d)), device=dev,
                         dtype=torch.uint8)
        fn = lambda: fox.attn_fwd_pruned(q, k, v, logf, scale=inp["scale"], out=o, lse=lse, c=c,  # noqa: E731
                                         workspace=ws)
    elif mode == "token":
        tm = lambda t: t.permute(0, 2, 1, 3).contiguous()  # noqa: E731
        q, k, v, logf = tm(q), tm(k), tm(v), logf.permute(0, 2, 1).contiguous()
        o, lse, c = torch.empty_like(q), torch.empty_like(logf), torch.empty_like(logf)
        fn = lambda: fox.attn_fwd_ex(q, k, v, logf, causal=True, layout="token", scale=inp["scale"],  # noqa: E731
                                     out=o, lse=lse, c=c)
    else:
        fn = lambda: fox.attn_fwd(q, k, v, logf, scale=inp["scale"], out=o, lse=lse, c=c)  # noqa: E731
    _warm(torch, fn, warmup)
    region = _events_time(torch, fn, steps)
    flops = 4.0 * cfg.d * cfg.N * cfg.N * cfg.B * cfg.H if mode == "unmasked" else fwd_flops(cfg)
    ms = region / steps
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = flops / (ms * 1e-3) / 1e12
    kernel = fwd_kernel_name(torch, cfg, causal=mode != "unmasked") + ({"unmasked": " unmasked", "pruned": " pruned",
                                             "token": " token-major"}.get(mode, ""))
    return {
        "cfg": cfg, "inp": inp,
        "ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
        "kernel": kernel, "launch_ms_mean": ms,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": stored_traffic(tag, kernel, "fwd")},
        "flop_per_launch": flops,
    }


def bench_bwd(torch, fox, fi, tag, steps, warmup, staged=False):
    """fox_attn_bwd on the forward workload `tag`: 10*d flop per causal pair (the recomputed
    q.k, and dP, dV, dK, dQ), timed whole (row-vector, key-side, query-side and scan kernels).
    staged: fox_attn_bwd_staged (bf16, d = 128), whose key side stores dS for the dQ contraction."""
    cfg = fi.FWD[tag]
    inp = fi.fwd_inputs(cfg)
    dev = "cuda"
    q, k, v, logf = (inp[n].to(dev) for n in ("q", "k", "v", "logf"))
    o, lse, c = fox.attn_fwd(q, k, v, logf, scale=inp["scale"])
    g = torch.Generator().manual_seed(1)
    dout = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dl = torch.empty_like(logf)
    if staged:
        ws = torch.empty(fox.attn_bwd_staged_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d), device=dev,
                         dtype=torch.uint8)
        fn = lambda: fox.attn_bwd_staged(q, k, v, o, dout, lse, logf, scale=inp["scale"], dq=dq, dk=dk,  # noqa: E731
                                         dv=dv, dlogf=dl, workspace=ws)
    else:
        ws = torch.empty(fox.attn_bwd_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d), device=dev, dtype=torch.uint8)
        fn = lambda: fox.attn_bwd(q, k, v, o, dout, lse, logf, scale=inp["scale"], dq=dq, dk=dk, dv=dv,  # noqa: E731
                                  dlogf=dl, workspace=ws)
    _warm(torch, fn, warmup)
    region = _events_time(torch, fn, steps)
    ms = region / steps
    flops = 2.5 * fwd_flops(cfg)
    achieved = flops / (ms * 1e-3) / 1e12
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    kernel = (f"bwd_kv_kernel<{cfg.d},causal> + bwd_dq_kernel<{cfg.d},causal> + 2 small kernels" if bf16 else
              f"bwd_f32_kv_kernel<{cfg.d},causal> + bwd_f32_dq_kernel<{cfg.d},causal> + 2 small kernels")
    label = BWD_KERNEL
    note = ("10*d flop per causal pair (the dq kernel's recomputation of S and dP, 4*d more, is not "
            "counted); one call = the row-vector, key-side, query-side and gate suffix-sum kernels"
            + ("" if bf16 else "; fp32 on the vector ALU, a parity-sized workload (latency-bound)"))
    if staged:
        kernel = f"bwd_kv_kernel<{cfg.d},causal,staged> + bwd_dq_staged_kernel<{cfg.d}> + 2 small kernels"
        label = BWD_STAGED_KERNEL
        note = ("10*d flop per causal pair; fox_attn_bwd_staged: the key side stores the bf16 dS "
                f"({ws.numel() / 1e9:.2f} GB of workspace) and dQ is contracted from it, no recomputation")
    traffic = stored_traffic(tag, label.format(d=cfg.d), "bwd") if bf16 else None
    return {"workload": cfg.desc + (", backward, staged dS" if staged else ", backward"), "value": round(achieved, 2),
            "unit": "TFLOP/s", "ms_per_step": round(ms, 4), "note": note,
            "roofline": {"bound": "mfma" if bf16 else "alu", "achieved": round(achieved, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel}}


_DECODE_INPUTS = {}


def bench_decode(torch, fox, fi, tag, steps, warmup, cache="plain"):
    """cache: "plain" (fox_attn_decode), "ragged" (fox_attn_decode_ragged, seeded lengths in
    [1, L]; bytes of the slots in use) or "paged" (fox_attn_decode_paged, every sequence at full
    length in 256-slot pages scattered over a shuffled pool; the same bytes as "plain")."""
    cfg = fi.DECODE[tag]
    t0 = time.time()
    if tag not in _DECODE_INPUTS:  # the host inputs are reused by the cache variants
        _DECODE_INPUTS.clear()
        _DECODE_INPUTS[tag] = fi.decode_inputs(cfg)
    inp = _DECODE_INPUTS[tag]
    gen_s = time.time() - t0
    dev = "cuda"
    L = cfg.L
    q = inp["q"].to(dev)
    kc = inp["k"].to(dev)
    vc = inp["v"].to(dev)
    cc = fox.logf_cumsum(inp["logf_all"].to(dev))  # the cache's prefix sums, built by the library's scan
    lnew = inp["logf_all"][..., L - 1].contiguous().to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(cfg.S, cfg.H, device=dev)
    ws = torch.empty(fox.decode_workspace_bytes(cfg.S, cfg.H, L, cfg.d), device=dev, dtype=torch.uint8)
    lens = None
    if cache == "ragged":
        g = torch.Generator().manual_seed(3)
        lens = torch.randint(1, L + 1, (cfg.S,), generator=g, dtype=torch.int32)
        ld = lens.to(dev)
        fn = lambda: fox.attn_decode_ragged(q, kc, vc, cc, lnew, ld, scale=inp["scale"], out=o, lse=lse,  # noqa
                                            workspace=ws)
    elif cache == "paged":
        P = 256
        maxp = L // P
        npages = cfg.S * maxp + 3
        g = torch.Generator().manual_seed(4)
        table = torch.randperm(npages, generator=g)[: cfg.S * maxp].to(torch.int32).reshape(cfg.S, maxp).to(dev)
        kp = torch.empty(npages, cfg.H, P, cfg.d, device=dev, dtype=kc.dtype)
        vp = torch.empty_like(kp)
        cp = torch.empty(npages, cfg.H, P, device=dev, dtype=torch.float32)
        flat = table.flatten().long()
        kp[flat] = kc.view(cfg.S, cfg.H, maxp, P, cfg.d).permute(0, 2, 1, 3, 4).reshape(-1, cfg.H, P, cfg.d)
        vp[flat] = vc.view(cfg.S, cfg.H, maxp, P, cfg.d).permute(0, 2, 1, 3, 4).reshape(-1, cfg.H, P, cfg.d)
        cp[flat] = cc.view(cfg.S, cfg.H, maxp, P).permute(0, 2, 1, 3).reshape(-1, cfg.H, P)
        del kc, vc
        kc = vc = None
        ld = torch.full((cfg.S,), L, dtype=torch.int32, device=dev)
        fn = lambda: fox.attn_decode_paged(q, kp, vp, cp, table, ld, lnew, scale=inp["scale"], out=o, lse=lse,  # noqa
                                           workspace=ws)
    else:
        fn = lambda: fox.attn_decode(q, kc, vc, cc, lnew, scale=inp["scale"], out=o, lse=lse, workspace=ws)  # noqa
    _warm(torch, fn, warmup)
    region = _events_time(torch, fn, steps)
    by = decode_bytes(cfg, lens)
    ms = region / steps
    achieved = by["total"] / (ms * 1e-3) / 1e9
    res = {
        "workload": cfg.desc + ("" if cache == "plain" else f", {cache} cache"), "ms_per_step": round(ms, 4),
        "value": round(by["total"] / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s", "bytes_per_step": by["total"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": stored_traffic(tag, DECODE_KERNEL, "decode") if cache == "plain" else None,
                     "kernel": DECODE_KERNEL if cache == "plain" else DECODE_KERNEL.replace(",128>", f",128,{cache}>"),
                     "note": "per call = split kernel + combine kernel; bytes = algorithmic bytes per call"},
        "input_gen_s": round(gen_s, 1),
    }
    del kc, vc
    return res, inp


def _blas_threads() -> int:
    """Threads the oracle's NumPy BLAS actually uses."""
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _host_info() -> dict:
    """The host the oracle runs on: logical CPUs, the ones this process may use, and the model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model,
            "blas_threads": _blas_threads()}


def sample_rows(n: int):
    """The oracle's row sample at long sequences: every 64th row of a head, plus its last 128 rows."""
    import numpy as np
    return np.unique(np.concatenate([np.arange(0, n, 64), np.arange(max(0, n - 128), n)]))


def cpu_baseline_fwd(fi, inp, budget_s=15.0, rows_sample=False):
    """The fp64 oracle, as it stands, on heads of the same workload: whole heads, or with
    rows_sample the rows of sample_rows() of every head, cycling over the heads until the budget
    is spent.  Its rate counts the algorithmic work of the rows done (4 d flop per causal pair)."""
    import numpy as np

    import oracle
    cfg = inp["cfg"]
    q, k, v, lf = (inp[n] for n in ("q", "k", "v", "logf"))
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    rows = sample_rows(cfg.N) if rows_sample else np.arange(cfg.N)
    pairs_per_head = float(np.sum(rows + 1))
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b, h = heads[done % len(heads)]
        oracle.fwd_head_rows(q[b, h].double().numpy(), k[b, h].double().numpy(), v[b, h].double().numpy(),
                             lf[b, h].double().numpy(), inp["scale"], rows)
        done += 1
    dt = time.perf_counter() - t0
    flops = 4.0 * cfg.d * pairs_per_head * done
    what = (f"rows {{0, 64, 128, ...}} and the last 128 ({len(rows)} of {cfg.N}) of each head" if rows_sample
            else f"all {cfg.N} rows of each head")
    info = _host_info()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"{done} (batch, head) slices of the same workload ({len(heads)} in all, cycled), {what}; "
                      f"fp64 NumPy, {dt:.1f} s wall; rate = the algorithmic flop of those rows / wall time",
            "host": info}


def cpu_baseline_decode(inp, cfg, budget_s=10.0):
    """The fp64 oracle's decode, as it stands, over whole sequences (all heads) until the budget is
    spent; bytes counted as the GPU's algorithmic bytes of those sequences."""
    import numpy as np

    import oracle
    L = cfg.L
    t0 = time.perf_counter()
    done = 0
    for s in range(inp["q"].shape[0]):
        lf = inp["logf_all"][s:s + 1].double().numpy()
        cc = oracle.logf_cumsum(lf).astype(np.float32).astype(np.float64)  # an fp32 cache, like the GPU's
        oracle.attn_decode(inp["q"][s:s + 1].double().numpy(), inp["k"][s:s + 1].double().numpy(),
                           inp["v"][s:s + 1].double().numpy(), cc, lf[..., L - 1], inp["scale"])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    by = decode_bytes(cfg)["total"] * done / cfg.S
    info = _host_info()
    return {"value": round(by / dt / 1e9, 3), "unit": "GB/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"{done} of {cfg.S} sequences (all {cfg.H} heads each), fp64 NumPy, {dt:.1f} s wall",
            "host": info}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "c2_f1", "c2_alibi", "c3", "c4", "c5"])
    ap.add_argument("--backward", action="store_true", help="with --only: time fox_attn_bwd on the workload")
    ap.add_argument("--staged", action="store_true", help="with --backward: time fox_attn_bwd_staged instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time a captured HIP graph of the K calls")
    ap.add_argument("--only", action="store_true", help="measure the selected workload only")
    ap.add_argument("--copy-calibration", action="store_true", help="run the 1 GiB device copy for counter scaling")
    ap.add_argument("--traffic-summary", action="store_true", help="write a traffic summary from counter CSVs")
    ap.add_argument("--fetch-csv"), ap.add_argument("--write-csv")
    ap.add_argument("--copy-fetch-csv"), ap.add_argument("--copy-write-csv")
    ap.add_argument("--kernel", help="kernel label as bench.py reports it"), ap.add_argument("--kernel-match")
    ap.add_argument("--kind", choices=["fwd", "decode", "bwd"], default="fwd")
    ap.add_argument("--alg-bytes", type=float, default=0.0), ap.add_argument("--out")
    ap.add_argument("--trace-summary", action="store_true", help="write a kernel-trace summary from a stats CSV")
    ap.add_argument("--stats-csv"), ap.add_argument("--bench-log"), ap.add_argument("--title")
    ap.add_argument("--bench-args", default=""), ap.add_argument("--note", action="append")
    ap.add_argument("--mfma-summary", action="store_true", help="write an MFMA-use summary from counter CSVs")
    ap.add_argument("--pmc-csv", action="append", help="workload:kind:path of one counter run")
    args = ap.parse_args()
    if args.trace_summary:
        write_trace_summary(args)
        return
    if args.mfma_summary:
        write_mfma_summary(args)
        return
    global USE_GRAPH
    USE_GRAPH = args.graph
    if args.traffic_summary:
        write_traffic_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU sharding is not built", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import forget_gated_causal_amd as fox
    import fox_inputs as fi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    print(f"# device: {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded, see fox_inputs.py)",
            "timing": ("the K calls captured in one HIP graph, replayed between two HIP events" if USE_GRAPH
                       else "K direct calls between two HIP events")}
    if args.workload == "c5":
        dec, dinp = bench_decode(torch, fox, fi, "c5", args.steps, args.warmup)
        line.update({"value": dec["value"], "unit": "GB/s", "ms_per_step": dec["ms_per_step"], "dtype": "bf16",
                     "config": {"workload": dec["workload"], "global_batch": 64, "seq_len": 8192,
                                "parallelism": "single GPU"},
                     "roofline": dec["roofline"]})
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_decode(dinp, fi.DECODE["c5"])
        print(json.dumps(line), flush=True)
        return

    if args.backward:
        x = bench_bwd(torch, fox, fi, args.workload, args.steps, args.warmup, staged=args.staged)
        print(f"# {x['workload']}: {x['ms_per_step']*1e3:.1f} us/step, {x['value']:.1f} TFLOP/s", file=sys.stderr,
              flush=True)
        line.update({"value": x["value"], "unit": "TFLOP/s", "ms_per_step": x["ms_per_step"],
                     "dtype": fi.FWD[args.workload].dtype, "config": {"workload": x["workload"]},
                     "roofline": x["roofline"]})
        print(json.dumps(line), flush=True)
        return
    r = bench_fwd(torch, fox, fi, args.workload, args.steps, args.warmup)
    cfg = r["cfg"]
    print(f"# {cfg.desc}: {r['ms_per_step']*1e3:.1f} us/step, {r['tflops']:.1f} TFLOP/s, {r['kernel']}",
          file=sys.stderr, flush=True)
    line.update({
        "value": round(r["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(r["ms_per_step"], 5),
        "dtype": cfg.dtype,
        "config": {"workload": cfg.desc + (" (the largest single-GPU forward configuration)" if args.workload == "c4"
                                           else ""),
                   "global_batch": cfg.B, "seq_len": cfg.N, "heads": cfg.H, "head_dim": cfg.d,
                   "parallelism": "single GPU"},
        "roofline": dict(r["roofline"], kernel=r["kernel"], launch_us_mean=round(r["launch_ms_mean"] * 1e3, 2),
                         flop_per_launch=r["flop_per_launch"]),
    })
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_fwd(fi, r["inp"], rows_sample=cfg.N >= 8192)
    del r
    torch.cuda.empty_cache()
    if not args.only:
        others = {}
        for tag in [t for t in ("c2", "c3", "c4") if t != args.workload]:
            x = bench_fwd(torch, fox, fi, tag, max(10, args.steps // 5), max(3, args.warmup // 2))
            print(f"# {x['cfg'].desc}: {x['ms_per_step']*1e3:.1f} us/step, {x['tflops']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
            others[tag] = {"workload": x["cfg"].desc, "value": round(x["tflops"], 2), "unit": "TFLOP/s",
                           "ms_per_step": round(x["ms_per_step"], 4),
                           "roofline": dict(x["roofline"], kernel=x["kernel"])}
            del x
            torch.cuda.empty_cache()
        for tag, mode in (("c2", "unmasked"), ("c3", "pruned"), ("c2", "token"), ("c3", "token")):
            x = bench_fwd(torch, fox, fi, tag, max(10, args.steps // 5), max(3, args.warmup // 2), mode=mode)
            print(f"# {x['cfg'].desc}, {mode}: {x['ms_per_step']*1e3:.1f} us/step, {x['tflops']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
            note = {"unmasked": "4*d flop for every (query, key) pair",
                    "pruned": "effective rate: the causal work over the time of the pruned call (key-norm, "
                              "prefix-sum and forward kernels); skipped keys weigh < 2^-24 of each row sum",
                    "token": "q, k, v, o as [B,N,H,d], logf, lse, c as [B,N,H]"}[mode]
            others[f"{tag}_{mode}"] = {"workload": x["cfg"].desc + f", {mode}", "value": round(x["tflops"], 2),
                                       "unit": "TFLOP/s", "ms_per_step": round(x["ms_per_step"], 4),
                                       "note": note, "roofline": dict(x["roofline"], kernel=x["kernel"])}
            del x
            torch.cuda.empty_cache()
        for tag in ("c1", "c2", "c3"):
            x = bench_bwd(torch, fox, fi, tag, max(10, args.steps // 5), max(3, args.warmup // 2))
            print(f"# {x['workload']}: {x['ms_per_step']*1e3:.1f} us/step, {x['value']:.1f} TFLOP/s", file=sys.stderr,
                  flush=True)
            others[f"{tag}_backward"] = x
            torch.cuda.empty_cache()
        x = bench_bwd(torch, fox, fi, "c3", max(10, args.steps // 5), max(3, args.warmup // 2), staged=True)
        print(f"# {x['workload']}: {x['ms_per_step']*1e3:.1f} us/step, {x['value']:.1f} TFLOP/s", file=sys.stderr,
              flush=True)
        others["c3_backward_staged"] = x
        del x
        torch.cuda.empty_cache()
        dec, dinp = bench_decode(torch, fox, fi, "c5", max(10, args.steps // 5), max(3, args.warmup // 2))
        print(f"# {dec['workload']}: {dec['ms_per_step']*1e3:.1f} us/step, {dec['value']:.0f} GB/s",
              file=sys.stderr, flush=True)
        if not args.no_cpu_baseline:
            dec["cpu_baseline"] = cpu_baseline_decode(dinp, fi.DECODE["c5"])
        others["c5_decode"] = dec
        torch.cuda.empty_cache()
        for cache in ("ragged", "paged"):
            x, _ = bench_decode(torch, fox, fi, "c5", max(10, args.steps // 5), max(3, args.warmup // 2), cache=cache)
            print(f"# {x['workload']}: {x['ms_per_step']*1e3:.1f} us/step, {x['value']:.0f} GB/s", file=sys.stderr,
                  flush=True)
            others[f"c5_{cache}"] = x
            torch.cuda.empty_cache()
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
