"""FLCE forward + backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --copy-probe BYTES          # one plain device copy of BYTES (counter calibration)
    python bench.py --summarize-trace DIR       # markdown table from a rocprofv3 --kernel-trace run
    python bench.py --summarize-pmc DIR         # markdown table from a rocprofv3 --pmc run
    python bench.py --summarize-alloc DIR       # device allocations from a --memory-allocation-trace run
    python bench.py --shards P                  # the vocabulary-shard path: P shards in sequence
    python bench.py --hbm-activity              # HBM-side activity of the FLCE calls (amdsmi)

A step is one pass of the whole hot path over one batch: flce_forward_keep
(logits GEMM with the online log-sum-exp epilogue, combine, reduction; the
first vocabulary slab's logits kept) then flce_backward_kept (that slab's
dlogits from the kept values; per other slab the logits recompute into
dlogits; per slab dx and dW; db), with inputs, outputs, workspaces and the
kept buffer already resident in HBM.  --schedule recompute times
flce_forward + flce_backward (every slab recomputed) instead.  Prints one
JSON line.  Inputs are seeded synthetic data with the workload's shapes and
distributions (random weights; no dataset).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FLCE fwd+bwd tokens/s and % bf16 MFMA peak at N=8192,H=4096,V=128256"


def metric_for(w):
    """The metric string of a workload: the headline's wording at its own shape
    (fp16 and fp32 inputs say so)."""
    m = f"FLCE fwd+bwd tokens/s and % bf16 MFMA peak at N={w.N},H={w.H},V={w.V}"
    if w.dtype == "f16":
        m += " (fp16 inputs; fp16 MFMA peak = bf16's)"
    elif w.dtype == "f32":
        m = f"FLCE fwd+bwd tokens/s and % fp32 MFMA peak at N={w.N},H={w.H},V={w.V}"
    return m


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (fp16 the same)
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 matrix


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0: automatic)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES")
    p.add_argument("--summarize-trace", default=None, metavar="DIR")
    p.add_argument("--summarize-pmc", default=None, metavar="DIR")
    p.add_argument("--summarize-alloc", default=None, metavar="DIR")
    p.add_argument("--hbm-activity", action="store_true",
                   help="memory-controller activity (amdsmi) while calibration loops and the FLCE calls run")
    p.add_argument("--shards", type=int, default=0, metavar="P",
                   help="time the vocabulary-shard entry points: W split into P shards run one after another")
    p.add_argument("--schedule", choices=("keep", "recompute", "fused"), default="keep",
                   help="keep: flce_forward_keep + flce_backward_kept (the recompute schedule with the first "
                        "vocabulary slab's logits kept from the forward; the headline); recompute: "
                        "flce_forward + flce_backward (every slab recomputed); fused: the gradients formed "
                        "in the forward pass (flce_fused_forward_backward)")
    p.add_argument("--chunk", type=int, default=0, help="fused schedule: tokens per chunk (0: equal memory)")
    p.add_argument("--no-fused-line", action="store_true",
                   help="leave the fused schedule's comparison out of the recompute line")
    p.add_argument("--no-kernel-times", action="store_true",
                   help="leave out the library's launch timing log (counter runs); roofline falls back to "
                        "the forward call")
    return p.parse_args()


def _code_only(text):
    """C++/HIP source with comments removed and whitespace collapsed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(sources=None):
    """Hash of the HIP sources' code (comments and whitespace ignored); a traffic
    figure is valid only for this hash.  ``sources``: {file name: text}, default
    the files under csrc/."""
    if sources is None:
        sources = {}
        for f in glob.glob(os.path.join(ROOT, "lm_head_cross_flce_amd", "csrc", "*")):
            with open(f, encoding="utf-8") as fh:
                sources[os.path.basename(f)] = fh.read()
    h = hashlib.sha256()
    for name in sorted(sources):
        h.update(name.encode() + _code_only(sources[name]).encode())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    from the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source hash: `([0-9a-f]+)`", text)
    t = re.search(r"traffic_bytes_per_launch: ([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def recorded_trace(kernel, workload):
    """The committed kernel trace of this workload, if it was taken from the
    current kernel sources: {"file", "avg_us"} for ``kernel`` (its average
    launch duration over every launch of the traced run), else None."""
    rel_path = os.path.join("profiles", f"flce_step_{workload}_kernel_trace.md")
    path = os.path.join(ROOT, rel_path)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"Source hash `([0-9a-f]+)`", text)
    names = [k.strip() for k in kernel.split("+")]
    avgs = []
    for k in names:
        a = re.search(r"kernel_avg_us: " + re.escape(k) + r" ([0-9.]+) over (\d+) launches", text)
        if not a:
            return None
        avgs.append(float(a.group(1)))
    if not m or m.group(1) != kernel_source_hash():
        return None
    return {"file": rel_path, "avg_us": sum(avgs)}


def _kernel_rows(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    rows = []
    if files:
        for f in files:
            for r in csv.DictReader(open(f)):
                rows.append((r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        return rows
    import sqlite3
    for db in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
        c = sqlite3.connect(db)
        rows += [(n, int(e) - int(s)) for n, s, e in c.execute("select name, start, end from kernels")]
    return rows


def summarize_trace(d):
    """Per kernel: launches, average duration, and the warm average that leaves
    out each kernel's first launch (cold caches and clocks)."""
    rows = _kernel_rows(d)
    agg = {}
    for name, dur in rows:
        key = name.split("(")[0].replace("void ", "")
        agg.setdefault(key, []).append(dur)
    total = sum(sum(v) for v in agg.values())
    print("| kernel | calls | avg us | warm avg us | total ms | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        t, n = sum(v), len(v)
        warm = (t - v[0]) / (n - 1) if n > 1 else t
        print(f"| `{k}` | {n} | {t / n / 1e3:.1f} | {warm / 1e3:.1f} | {t / 1e6:.2f} | {100 * t / total:.1f}% |")
    # Per kernel over all its template instances: the average launch duration
    # that the benchmark's roofline compares with its live figure.
    fam = {}
    for k, v in agg.items():
        f = k.replace("flce::", "").split("<")[0]
        fam.setdefault(f, []).extend(v)
    print()
    for f, v in sorted(fam.items(), key=lambda kv: -sum(kv[1])):
        print(f"kernel_avg_us: {f} {sum(v) / len(v) / 1e3:.2f} over {len(v)} launches")


def summarize_alloc(d):
    """Device allocations of a rocprofv3 --memory-allocation-trace run, 1 MB and up."""
    files = glob.glob(os.path.join(d, "**", "*memory_allocation_trace.csv"), recursive=True)
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            size = int(r.get("Allocation_Size", 0) or 0)
            if size >= 1 << 20:
                rows.append((int(r.get("Start_Timestamp", 0) or 0), r.get("Operation", "?"), size,
                             r.get("Agent_Type", r.get("Agent_Id", ""))))
    rows.sort()
    total = 0
    print("| # | operation | bytes | MB |")
    print("|---:|---|---:|---:|")
    for i, (_, op, size, _) in enumerate(rows):
        total += size if "FREE" not in op.upper() else 0
        print(f"| {i} | {op} | {size} | {size / 1e6:.1f} |")
    print(f"\nallocated (1 MB and up, frees not subtracted): {total / 1e6:.1f} MB")


def summarize_pmc(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    agg, disp = {}, {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"].split("(")[0].replace("void ", ""), r["Counter_Name"])
            agg[key] = agg.get(key, 0.0) + float(r["Counter_Value"])
            disp.setdefault(key[0], set()).add(r["Dispatch_Id"])
    print("| kernel | counter | per dispatch | dispatches |")
    print("|---|---|---:|---:|")
    for (k, c), v in sorted(agg.items()):
        n = len(disp[k])
        print(f"| `{k}` | {c} | {v / n:.6g} | {n} |")


def copy_probe(nbytes):
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": a.numel() * 4, "copy_probe_bytes_written": b.numel() * 4}))


def refresh_window_activity(refreshes):
    """Average memory-controller busy percentage over consecutive refreshes of
    the gpu metrics table.  ``refreshes``: (system_clock_counter ns,
    mem_activity_acc) per refresh, in order, every one seen after the loop
    started and before it ended.  The window ending at the first refresh began
    before the loop, so only the windows between refreshes count.  Returns
    (percent or None, windows, their total length in ms)."""
    pairs = list(zip(refreshes, refreshes[1:]))
    acc = sum(b[1] - a[1] for a, b in pairs)
    span_ms = sum(b[0] - a[0] for a, b in pairs) * 1e-6
    return (acc / span_ms if span_ms > 0 else None), len(pairs), span_ms


def hbm_activity(F, w, x, W, b, tg, g, seconds=4.0):
    """Memory-controller activity while loops of known HBM traffic run, then
    while the FLCE calls run.

    The L2 fetch counters count every L2 miss, including those that the 256 MB
    last-level cache in front of HBM serves.  The SMU's gpu metrics table
    (amdsmi) sees only the memory controllers: `mem_activity_acc` adds their
    busy percentage every millisecond, and the table is refreshed about once a
    second together with `system_clock_counter` (ns).  Each phase keeps its
    loop on the GPU for ``seconds`` and averages the refresh windows that lie
    wholly inside it: percent = sum of acc deltas / sum of clock deltas (ms).
    A read-only loop over 2 GiB (larger than that cache) gives percent per
    TB/s; a loop re-reading 128 MiB (which fits it) is the control.  Each phase
    prints one JSON line; the FLCE calls add the HBM bytes per call that the
    read calibration implies."""
    import threading
    import torch
    import amdsmi

    amdsmi.amdsmi_init()
    try:
        h = amdsmi.amdsmi_get_processor_handles()[0]
        dev = x.device
        N, H, V = w.N, w.H, w.V

        def table():
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            return (m["system_clock_counter"], m["mem_activity_acc"], m["average_umc_activity"],
                    m["current_gfxclk"])

        def phase(name, fn, nbytes=None):
            print(f"[hbm-activity] {name}", file=sys.stderr, flush=True)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fn()
            e0.record()
            for _ in range(3):
                fn()
            e1.record()
            torch.cuda.synchronize()
            iters = max(4, int(seconds * 1e3 / (e0.elapsed_time(e1) / 3)))
            seen, stop = [], threading.Event()
            base = table()[0]

            def poll():
                last = base
                while not stop.is_set():
                    t = table()
                    if t[0] != last:   # a refresh: (host time seen, clock, acc, average, gfxclk)
                        seen.append((time.perf_counter(),) + t)
                        last = t[0]
                    time.sleep(0.02)

            th = threading.Thread(target=poll)
            th.start()
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t_end = time.perf_counter()
            stop.set()
            th.join()
            ms = e0.elapsed_time(e1) / iters
            inside = [s for s in seen if s[0] < t_end - 0.05]
            pct, windows, span_ms = refresh_window_activity([(s[1], s[2]) for s in inside])
            r = {"phase": name, "iters": iters, "ms_per_iter": ms, "windows": windows, "window_ms": span_ms,
                 "umc_activity_pct": pct, "average_umc_activity": [s[3] for s in inside[1:]],
                 "gfxclk_mhz": [s[4] for s in inside[1:]]}
            if nbytes:
                r["bytes_per_iter"] = nbytes
                r["tb_per_s"] = nbytes / (ms * 1e-3) / 1e12
            return r

        def emit(r):
            print(json.dumps(r), flush=True)

        emit(phase("idle", lambda: torch.cuda._sleep(20_000_000)))
        big = torch.ones((2 << 30) // 4, dtype=torch.float32, device=dev)
        cal = phase("read 2 GiB", lambda: torch.sum(big), big.numel() * 4)
        emit(cal)
        small = big[: (128 << 20) // 4]
        emit(phase("read 128 MiB (fits the last-level cache)", lambda: torch.sum(small), small.numel() * 4))
        dst = torch.empty_like(big)
        emit(phase("copy 2 GiB", lambda: dst.copy_(big), 2 * big.numel() * 4))
        del big, small, dst
        torch.cuda.empty_cache()
        pct_per_tbps = cal["umc_activity_pct"] / cal["tb_per_s"]

        fb, kb, bb = F.flce_keep_workspace_size(N, H, V, x.dtype, b is not None, w.reduction)
        rfb, rbb = F.flce_workspace_size(N, H, V, x.dtype, b is not None, w.reduction)
        ws_f = torch.empty(max(fb, rfb), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(max(bb, rbb), dtype=torch.uint8, device=dev)
        kbuf = torch.empty(kb, dtype=torch.uint8, device=dev)
        outs = (torch.empty_like(x), torch.empty_like(W), torch.empty_like(b) if b is not None else None)
        args = (w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
        _, lse, nv = F.flce_forward(x, W, b, tg, *args, workspace=ws_f)
        algo_fwd = (N * H + V * H) * x.element_size() + (V * b.element_size() if b is not None else 0) + N * 8

        def keep_step():
            _, lse_k, nv_k, _ = F.flce_forward_keep(x, W, b, tg, *args, workspace=ws_f, keep=kbuf)
            F.flce_backward_kept(x, W, b, tg, lse_k, nv_k, g, kbuf, *args, workspace=ws_b, out=outs)

        calls = [
            ("forward, every vocabulary column (flce_forward)",
             lambda: F.flce_forward(x, W, b, tg, *args, workspace=ws_f), algo_fwd),
            ("backward, every slab recomputed (flce_backward)",
             lambda: F.flce_backward(x, W, b, tg, lse, nv, g, *args, workspace=ws_b, out=outs), None),
            ("step, first slab kept (flce_forward_keep + flce_backward_kept)", keep_step, None),
        ]
        for name, fn, algo in calls:
            r = phase(name, fn)
            if r["umc_activity_pct"] is not None:
                r["hbm_bytes_per_iter_est"] = r["umc_activity_pct"] / pct_per_tbps * 1e12 * r["ms_per_iter"] * 1e-3
            if algo:
                r["algorithmic_bytes"] = algo
            emit(r)
        emit({"workload": f"N={N} H={H} V={V}", "calibration_pct_per_tb_per_s": pct_per_tbps})
    finally:
        amdsmi.amdsmi_shut_down()


def cpu_baseline(inp, rows):
    """Time the fp64 oracle (as it stands) on the first ``rows`` tokens."""
    import numpy as np
    from lm_head_cross_flce_amd import synth
    from oracle import flce_oracle as O

    w = inp.w
    W64 = inp.as_f64("W")
    b64 = inp.as_f64("b")
    x = synth.bf16_bits_to_f64(inp.x[:rows]) if w.dtype == "bf16" else inp.x[:rows].astype(np.float64)
    t = inp.targets[:rows]
    g = inp.grad[:rows] if w.reduction == "none" else inp.grad
    t0 = time.perf_counter()
    O.loss_and_grads(x, W64, b64, t, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                     rows_per_chunk=rows)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": rows / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"first {rows} of {w.N} tokens, full V={w.V} and H={w.H}, fp64 forward+backward "
                      f"(logits computed twice), {dt:.2f} s"}


def shard_bench(args, w, x, W, b, tg, g, name):
    """A step of the shard path: P shard forwards, the merge, P shard backwards
    summing the fp32 dx partials into one buffer (the cross-GPU sum and the final
    cast of dx are the caller's and are not timed)."""
    import torch
    from lm_head_cross_flce_amd import functional as F

    N, H, V, P = w.N, w.H, w.V, args.shards
    cuts = [k * V // P for k in range(P + 1)]
    dev = x.device
    shards = [(a, e, W[a:e], b[a:e] if b is not None else None) for a, e in zip(cuts[:-1], cuts[1:])]
    sizes = [F.flce_shard_workspace_size(N, H, e - a, x.dtype, b is not None) for a, e, _, _ in shards]
    ws_f = torch.empty(max(s[0] for s in sizes), dtype=torch.uint8, device=dev)
    ws_m = torch.empty(max(s[1] for s in sizes), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(s[2] for s in sizes), dtype=torch.uint8, device=dev)
    dx = torch.empty(N, H, dtype=torch.float32, device=dev)

    def step():
        stats = torch.stack([F.flce_shard_forward(x, Ws, bs, tg, a, V, w.label_smoothing, w.ignore_index,
                                                  workspace=ws_f) for a, e, Ws, bs in shards])
        loss, lse, nv = F.flce_shard_merge(stats, tg, V, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                           w.reduction, workspace=ws_m)
        for k, (a, e, Ws, bs) in enumerate(shards):
            F.flce_shard_backward(x, Ws, bs, tg, a, V, lse, nv, g, w.label_smoothing, w.z_loss_scale,
                                  w.ignore_index, w.reduction, dx_partial=dx, accumulate_dx=k > 0,
                                  workspace=ws_b)
        return loss

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        loss = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    tflops = 8.0 * N * H * V / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": f"FLCE fwd+bwd tokens/s, vocabulary split into {P} shards run in sequence on one GPU",
        "value": N * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": w.dtype,
        "data": "synthetic (seeded SplitMix64 draws, random-init weights)",
        "config": {"workload": name, "N": N, "H": H, "V": V, "shards": P, "shard_rows": cuts[1] - cuts[0]},
        "tflops_8nhv": tflops, "mfma_frac_8nhv": tflops / PEAK_BF16_TFLOPS,
        "loss": loss.sum().item() if loss.numel() > 1 else loss.item(),
        "workspace_mb": (ws_f.numel() + ws_m.numel() + ws_b.numel()) / 1e6,
    }), flush=True)


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.summarize_alloc:
        summarize_alloc(args.summarize_alloc)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path would shard "
              "tokens across GPUs with a dW reduce-scatter, which this library does not implement)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lm_head_cross_flce_amd import _lib, functional as F, synth

    if not os.path.exists(_lib.LIB_PATH):
        from lm_head_cross_flce_amd import build
        build.build()
    name = args.workload or synth.BENCH_WORKLOAD
    w = synth.WORKLOADS[name]
    t_gen = time.perf_counter()
    inp = synth.make_inputs(w)
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {name}: inputs drawn in {t_gen:.1f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(w.dtype, torch.float32)

    def t(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, W = t(inp.x), t(inp.W)
    b = t(inp.b) if inp.b is not None else None
    tg = torch.from_numpy(inp.targets).to(dev)
    g = torch.from_numpy(inp.grad).to(dev)
    N, H, V = w.N, w.H, w.V
    torch.cuda.synchronize()
    mem_inputs = torch.cuda.memory_allocated(dev)   # x, W, b, targets, upstream grad
    keep_mode = args.schedule == "keep"
    if keep_mode:
        fwd_bytes, keep_bytes, bwd_bytes = F.flce_keep_workspace_size(N, H, V, tdt, b is not None, w.reduction)
    else:
        (fwd_bytes, bwd_bytes), keep_bytes = F.flce_workspace_size(N, H, V, tdt, b is not None, w.reduction), 0
    ws_f = torch.empty(fwd_bytes, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bwd_bytes, dtype=torch.uint8, device=dev)
    kbuf = torch.empty(keep_bytes, dtype=torch.uint8, device=dev) if keep_mode else None
    dx, dW = torch.empty_like(x), torch.empty_like(W)
    db = torch.empty_like(b) if b is not None else None
    stream = torch.cuda.current_stream(dev)

    if args.hbm_activity:
        del ws_f, ws_b, kbuf
        torch.cuda.empty_cache()
        hbm_activity(F, w, x, W, b, tg, g)
        return
    if args.shards > 0:
        shard_bench(args, w, x, W, b, tg, g, name)
        return
    if args.schedule == "fused":
        del ws_f, ws_b
        torch.cuda.empty_cache()
        r = fused_bench(F, w, (x, W, b, tg, g), (dx, dW, db), args.chunk, args.warmup, args.steps)
        peak = PEAK_BF16_TFLOPS if w.dtype in ("bf16", "f16") else PEAK_F32_TFLOPS
        ms = r["ms_per_step"]
        print(json.dumps({
            "metric": (METRIC if name == synth.BENCH_WORKLOAD else metric_for(w)) + ", fused schedule",
            "value": N * 1e3 / ms, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic (seeded SplitMix64 draws, random-init weights)",
            "config": {"workload": name, "N": N, "H": H, "V": V, "schedule": "fused", "chunk": r["chunk"]},
            "tflops_8nhv": 8.0 * N * H * V / (ms * 1e-3) / 1e12,
            "mfma_frac_8nhv": 8.0 * N * H * V / (ms * 1e-3) / 1e12 / peak,
            "tflops_6nhv": 6.0 * N * H * V / (ms * 1e-3) / 1e12,
            "extra_hbm_mb": r["extra_hbm_mb"], "extra_hbm_frac_of_fp32_logits": r["extra_hbm_mb"] * 1e6 / (N * V * 4.0),
            "loss": r["loss"],
        }), flush=True)
        return

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if keep_mode:
            loss, lse, nv, _ = F.flce_forward_keep(x, W, b, tg, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                                   w.reduction, workspace=ws_f, keep=kbuf)
        else:
            loss, lse, nv = F.flce_forward(x, W, b, tg, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                           w.reduction, workspace=ws_f)
        if ev is not None:
            ev[1].record(stream)
        if keep_mode:
            F.flce_backward_kept(x, W, b, tg, lse, nv, g, kbuf, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                 w.reduction, workspace=ws_b, out=(dx, dW, db))
        else:
            F.flce_backward(x, W, b, tg, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                            w.reduction, workspace=ws_b, out=(dx, dW, db))
        if ev is not None:
            ev[2].record(stream)
        return loss

    torch.cuda.reset_peak_memory_stats(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    if not args.no_kernel_times:
        _lib.flce_timing_start(128 * args.steps + 64)   # HIP events between the library's launches
    t0 = time.perf_counter()
    for k in range(args.steps):
        loss = step(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if not args.no_kernel_times:
        _lib.flce_timing_stop()
        launch_log = _lib.flce_timing_log()
        _lib.flce_timing_clear()
    # Measured extra memory: the allocator's peak over the warmup and timed steps, less
    # the inputs and the gradient outputs (dx, dW, db): the workspaces plus the
    # per-call loss, lse and count.
    out_bytes = sum(t_.numel() * t_.element_size() for t_ in (dx, dW, db) if t_ is not None)
    extra_measured = torch.cuda.max_memory_allocated(dev) - mem_inputs - out_bytes
    fwd_ms = sorted(e[0].elapsed_time(e[1]) for e in events)
    bwd_ms = sorted(e[1].elapsed_time(e[2]) for e in events)
    fwd_med, bwd_med = fwd_ms[len(fwd_ms) // 2], bwd_ms[len(bwd_ms) // 2]
    fwd_avg, bwd_avg = sum(fwd_ms) / len(fwd_ms), sum(bwd_ms) / len(bwd_ms)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = N * args.steps / elapsed
    flops = 8.0 * N * H * V
    peak = PEAK_BF16_TFLOPS if w.dtype in ("bf16", "f16") else PEAK_F32_TFLOPS
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    extra = fwd_bytes + keep_bytes + bwd_bytes + N * 4 + 8
    loss_v = loss.sum().item() if loss.numel() > 1 else loss.item()   # reduction none: report the sum
    print(f"[bench] loss {loss_v:.6f}; fwd {fwd_med:.3f} ms, bwd {bwd_med:.3f} ms (median)",
          file=sys.stderr, flush=True)

    if args.no_kernel_times:
        tf = 2.0 * N * H * V / (fwd_avg * 1e-3) / 1e12
        kernels = {"forward call": {"avg_us": fwd_avg * 1e3, "launches_per_step": 1, "ms_per_step": fwd_avg,
                                    "flops_per_launch": 2.0 * N * H * V, "tflops": tf, "frac": tf / peak,
                                    "method": "2NHV / the forward call's average duration from HIP events on "
                                              "the launch stream (no launch timing log)"}}
    else:
        code = {"bf16": _lib.FLCE_BF16, "f16": _lib.FLCE_F16, "f32": _lib.FLCE_F32}[w.dtype]
        slab = _lib.flce_backward_slab_cols(N, H, V, code)
        kernels = kernel_figures(launch_log, args.steps, N, H, V, min(slab, V) if keep_mode else 0, peak)
    gemms = {k: v for k, v in kernels.items() if "frac" in v}
    dominant = max(gemms, key=lambda k: gemms[k]["ms_per_step"])
    kd = kernels[dominant]
    print(f"[bench] per kernel: " + ", ".join(f"{k} {v['avg_us']:.1f} us x {v['launches_per_step']:g} "
                                              f"({100 * v['frac']:.1f}%)" for k, v in gemms.items()),
          file=sys.stderr, flush=True)

    out = {
        "metric": METRIC if name == synth.BENCH_WORKLOAD else metric_for(w),
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded SplitMix64 draws, random-init weights)",
        "config": {"workload": name, "N": N, "H": H, "V": V, "schedule": args.schedule, "bias": b is not None,
                   "label_smoothing": w.label_smoothing, "z_loss_scale": w.z_loss_scale,
                   "reduction": w.reduction, "ignored_rows": w.n_ignored, "targets": w.targets},
        "fwd_ms": fwd_med,
        "bwd_ms": bwd_med,
        "tflops_8nhv": tflops,
        "mfma_frac_8nhv": tflops / peak,
        "extra_hbm_mb": extra / 1e6,
        "extra_hbm_frac_of_fp32_logits": extra / (N * V * 4.0),
        "extra_hbm_measured_mb": extra_measured / 1e6,
        "keep_mb": keep_bytes / 1e6,
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": kd["tflops"], "peak": peak,
                     "unit": "TFLOP/s", "frac": kd["frac"], "traffic": recorded_traffic(dominant, name),
                     "avg_launch_us": kd["avg_us"], "flops_per_launch": kd["flops_per_launch"],
                     "note": kd["method"], "profile": profile_figure(dominant, name, kd, peak)},
        "kernels": kernels,
    }
    if not args.no_fused_line:
        ws_f = ws_b = kbuf = None
        torch.cuda.empty_cache()
        r = fused_bench(F, w, (x, W, b, tg, g), (dx, dW, db), 0, 1, max(3, args.steps // 2))
        r["mfma_frac_8nhv"] = 8.0 * N * H * V / (r["ms_per_step"] * 1e-3) / 1e12 / peak
        out["fused_schedule"] = r
        print(f"[bench] fused schedule: {r['ms_per_step']:.3f} ms per step, chunk {r['chunk']}, "
              f"{r['extra_hbm_mb']:.1f} MB", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        del x, W, b, dx, dW, db
        ws_f = ws_b = kbuf = None
        torch.cuda.empty_cache()
        rows = args.cpu_rows or max(8, min(N, int(1.8e13 // (8.0 * H * V))))   # ~15 s on 16 host threads
        print(f"[bench] cpu oracle on {rows} rows", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, rows)
    print(json.dumps(out), flush=True)


def profile_figure(kernel, workload, kd, peak):
    """The roofline figure recomputed from the committed trace of the same
    sources (its average launch duration), beside the live one; None without
    such a trace.  A kernel named "a + b" is one call of both kernels."""
    t = recorded_trace(kernel, workload)
    if t is None:
        return None
    tf = kd["flops_per_launch"] / (t["avg_us"] * 1e-6) / 1e12
    return {"file": t["file"], "avg_launch_us": t["avg_us"], "achieved": tf, "frac": tf / peak}


def fused_bench(F, w, inputs, outs, chunk, warmup, steps):
    """The fused schedule (gradients formed in the forward pass) on the same
    inputs and outputs: ms per step from HIP events on the launch stream, the
    chunk, and its extra memory (workspace plus loss, lse and count)."""
    import torch

    x, W, b, tg, g = inputs
    N, H, V = w.N, w.H, w.V
    nbytes, used = F.flce_fused_workspace_size(N, H, V, x.dtype, b is not None, chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)

    def step():
        return F.flce_fused_forward_backward(x, W, b, tg, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                             w.reduction, chunk_tokens=chunk, workspace=ws, out=outs)[0]

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        loss = step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del ws
    return {"ms_per_step": ms, "chunk": used, "extra_hbm_mb": (nbytes + N * 4 + 8) / 1e6,
            "loss": loss.sum().item() if loss.numel() > 1 else loss.item(),
            "method": "flce_fused_forward_backward, HIP events on the launch stream over the timed steps"}


def kernel_figures(log, steps, N, H, V, kept_cols, peak):
    """Per GEMM kernel, from the library's launch timing log over the timed
    steps (a HIP event on the launch stream before and after every launch):
    launches per step, average launch duration, and flops per launch = the
    kernel's flops per step / its launches per step.  Flops per step: the
    forward product 2NH(V - kept) (fwd_lse_kernel; kept = the first slab's
    columns when the forward keeps them, else 0), the kept-value forward
    2NH kept (fused_fwd_kernel), the recompute 2NH(V - kept) (bwd_dz_kernel),
    dx and dW 2NHV each.  The other kernels are listed with their time only."""
    gemm = {"fwd_lse_kernel": 2.0 * N * H * (V - kept_cols), "fused_fwd_kernel": 2.0 * N * H * kept_cols,
            "bwd_dz_kernel": 2.0 * N * H * (V - kept_cols), "bwd_dx_kernel": 2.0 * N * H * V,
            "bwd_dw_kernel": 2.0 * N * H * V}
    times = {}
    for name, ms in log:
        times.setdefault(name.strip("() ").split("<")[0].strip(), []).append(ms)
    out = {}
    for k, v in sorted(times.items(), key=lambda kv: -sum(kv[1])):
        n = len(v) / steps
        avg = sum(v) / len(v)
        row = {"avg_us": avg * 1e3, "launches_per_step": n, "ms_per_step": sum(v) / steps}
        if k in gemm and gemm[k] > 0:
            fl = gemm[k] / n
            tf = fl / (avg * 1e-3) / 1e12
            row.update({"flops_per_launch": fl, "tflops": tf, "frac": tf / peak,
                        "method": "flops per launch / average launch duration; durations from HIP events the "
                                  "library records on the launch stream around each launch (flce_timing_*) "
                                  "over the timed steps"})
        out[k] = row
    return out


if __name__ == "__main__":
    main()
