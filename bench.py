"""Benchmark of the MoE expert-parallel dispatch/combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]

One step is one pass of the whole hot path over one batch of the
DeepSeek-V3-shaped share (T=4096 tokens, H=7168 bf16, 256 experts over 8
segments, top-8, alignment 128), inputs resident in HBM:

    ep_dispatch_layout  -> ep_dispatch (bf16) -> ep_dispatch_nvfp4
    -> ep_combine -> ep_combine_bwd -> ep_dispatch_bwd

K steps are launched op by op through the Python binding and timed between
two device synchronizations; the host enqueues a step in about a third of
its GPU time, so the kernels run back to back.  The same step captured as
one HIP graph and replayed K times is reported as graph_ms_per_step (each
replay adds the graph launch's idle gap).  Each op is also captured as a graph of 8
back-to-back launches and bracketed by HIP events on the stream it runs on,
which gives each kernel's average duration.  Prints ONE JSON line on stdout:
tokens/s of the whole step (`value`), the roofline of the dominant kernel
(algorithmic bytes of one launch / its average duration, against the 8 TB/s
HBM peak), and the CPU oracle's tokens/s on the same batch (`cpu_baseline`).

--copy-calibration runs only a plain row copy of known size through the
dispatch kernel (identity routing, K=1): the reference for scaling the
rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
COLD_REPS = 20
MIN_OP_REPS = 50        # timed repetitions per op, whatever --steps is
METRIC = "dispatch+combine tokens/s and effective HBM GB/s (% of peak), 1 MI355X"
KERNEL_SOURCES = ("combine_ep_dispatch_amd/csrc/move.hip", "combine_ep_dispatch_amd/csrc/nvfp4.hip",
                  "combine_ep_dispatch_amd/csrc/layout.hip", "combine_ep_dispatch_amd/csrc/fp8.hip",
                  "combine_ep_dispatch_amd/csrc/nvfp4_combine.hip", "combine_ep_dispatch_amd/csrc/api.hip",
                  "combine_ep_dispatch_amd/csrc/epx_device.h", "combine_ep_dispatch_amd/csrc/nvfp4_device.h",
                  "combine_ep_dispatch_amd/csrc/fp8_device.h")


# Each layout path forced (timed beside the default choice; results must agree).
LAYOUT_PATHS = {"layout_lookback": 2, "layout_barrier": 8, "layout_two_kernel": 4, "layout_count": 16}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    """Digest of the kernel sources' code: comments and whitespace do not
    count, so editing a comment keeps the measured traffic valid."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


WORKLOAD_TITLES = {"dsv3": "DeepSeek-V3-shaped share", "tiny": "tiny", "skewed": "skewed routing (Zipf 1.2)",
                   "nvfp4": "NVFP4 dispatch with a fused shared expert",
                   "capacity": "capacity overflow (Zipf 1.5)"}


def traffic_for(op: str, workload: str):
    """HBM bytes per launch of `op` measured with rocprofv3 counters on
    `workload` (see profiles/), or None when missing, taken on another
    workload or on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("workload") != workload or doc.get("source_digest") != source_digest():
        return None
    entry = doc.get("ops", {}).get(op)
    return None if entry is None else entry.get("bytes_per_launch")


def in_step_for(workload: str):
    """Per-op durations inside the timed back-to-back steps, from the rocprofv3
    kernel trace of `workload` (see profiles/), or None when missing, taken
    on another workload or on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("workload") != workload or doc.get("source_digest") != source_digest():
        return None
    return doc


def algorithmic_bytes(w, kept: int, used_rows: int, kept_routed: int = None) -> dict:
    """Bytes each op must move at minimum: valid rows only, x read once,
    pad rows never touched (layout metadata: 12 bytes per used row)."""
    kept_routed = kept if kept_routed is None else kept_routed
    T, H, K, Kp = w.T, w.H, w.K, w.Kp
    row = 2 * H
    return {
        "layout": 4 * T * K + 4 * T * Kp + 12 * used_rows,
        "dispatch": row * T + row * kept + 4 * T * Kp,
        "dispatch_nvfp4": row * T + kept * (H // 2 + H // 16 + 2) + 4 * T * Kp,
        "combine": row * kept + row * T + 4 * T * K + 4 * T * Kp,
        "combine_bwd": row * T + row * kept + 4 * T * K + 4 * T * Kp,
        "dispatch_bwd": row * kept + row * T + 4 * T * Kp,
        # not part of the step: each layout path forced, the router-probability
        # gradient and FP8 dispatch
        "layout_lookback": 4 * T * K + 4 * T * Kp + 12 * used_rows,
        "layout_barrier": 4 * T * K + 4 * T * Kp + 12 * used_rows,
        "layout_two_kernel": 4 * T * K + 4 * T * Kp + 12 * used_rows,
        "layout_count": 4 * T * K + 4 * T * Kp + 12 * used_rows,
        "combine_bwd_probs": row * T + row * kept_routed + 4 * T * Kp + 4 * T * K,
        "dispatch_fp8": row * T + kept * (H + 4 * (H // 128)) + 4 * T * Kp,
        "combine_nvfp4": kept * (H // 2 + H // 16 + 2) + row * T + 4 * T * K + 4 * T * Kp,
    }


def cpu_baseline(w, host) -> dict:
    """Time the CPU oracle (single-threaded C) over the whole step on the same
    batch; tokens/s = T / seconds."""
    import oracle as orc

    orc.build(force=False)
    oc = orc.Cfg(T=w.T, H=w.H, E=w.E, S=w.S, K=w.K, A=w.align, C=w.capacity, shared=w.shared_expert,
                 src_seg=w.src_segment, recv_rows=host["R"])
    runs = []
    for _ in range(3):  # median of 3
        t0 = time.perf_counter()
        L = orc.layout(oc, host["ids"])
        tr = L["token_row"]
        res = {"layout": L, "recv": orc.dispatch(oc, tr, host["x"]),
               "nvfp4": orc.dispatch_nvfp4(oc, tr, host["x"]),
               "y": orc.combine(oc, tr, host["out"], host["probs"]),
               "gout": orc.combine_bwd(oc, tr, host["gy"], host["probs"]),
               "gx": orc.dispatch_bwd(oc, tr, host["grad_recv"])}
        runs.append(time.perf_counter() - t0)
    dt = statistics.median(runs)
    host["oracle_results"] = res
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(w.T / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"one full step (layout, bf16 + NVFP4 dispatch, combine, both backward passes) "
                      f"over the whole {w.T}-token batch, single-threaded C oracle, median of 3 runs {dt:.2f} s; "
                      f"host {cpu}, os.cpu_count()={os.cpu_count()}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--latency-sweep", default="",
                    help="comma-separated token counts: print per-op latency of the workload's "
                         "shape at each (small-batch serving), instead of the benchmark line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the work; --gpus {args.gpus} is not supported "
              "(destination ranks are modelled as segments of one receive buffer, no inter-GPU traffic)",
              file=sys.stderr)
        return 2

    import torch

    import combine_ep_dispatch_amd as epx
    from combine_ep_dispatch_amd import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        return copy_calibration(torch, epx, dev)
    if args.latency_sweep:
        return latency_sweep(torch, epx, wl, dev, args.workload, [int(v) for v in args.latency_sweep.split(",")])

    w = wl.CONFIGS[args.workload]
    log(f"[bench] workload {wl.describe(w)}")
    d = wl.make_workload(w)
    cfg = epx.EpConfig(num_tokens=w.T, hidden=w.H, num_experts=w.E, num_segments=w.S, top_k=w.K,
                       align=w.align, seg_capacity=w.capacity, shared_expert=w.shared_expert,
                       src_segment=w.src_segment)
    q = epx.ep_query(cfg)
    cfg.recv_rows = q.min_recv_rows
    R, T, H = cfg.recv_rows, w.T, w.H

    # inputs resident in HBM
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(d["topk_ids"].reshape(-1)).to(dev)
    probs = torch.from_numpy(d["probs"].reshape(-1)).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    out = torch.randn(R * H, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    gy = torch.randn(T * H, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    grad_recv = torch.randn(R * H, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    # outputs
    lay = epx.Layout.empty(cfg, dev)
    ws = epx.workspace_for(cfg, dev)
    recv = torch.empty(R * H, dtype=torch.bfloat16, device=dev)
    codes = torch.empty(R * H // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(R * H // 16, dtype=torch.uint8, device=dev)
    rowscale = torch.empty(R, dtype=torch.bfloat16, device=dev)
    y = torch.empty(T * H, dtype=torch.bfloat16, device=dev)
    gout = torch.empty(R * H, dtype=torch.bfloat16, device=dev)
    gx = torch.empty(T * H, dtype=torch.bfloat16, device=dev)

    ops = [
        ("layout", lambda: epx.ep_dispatch_layout(cfg, ids, ws, lay)),
        ("dispatch", lambda: epx.ep_dispatch(cfg, lay, x, recv)),
        ("dispatch_nvfp4", lambda: epx.ep_dispatch_nvfp4(cfg, lay, x, codes, scales, rowscale)),
        ("combine", lambda: epx.ep_combine(cfg, lay, out, probs, y)),
        ("combine_bwd", lambda: epx.ep_combine_bwd(cfg, lay, gy, probs, gout)),
        ("dispatch_bwd", lambda: epx.ep_dispatch_bwd(cfg, lay, grad_recv, gx)),
    ]
    names = [n for n, _ in ops]
    gprobs = torch.empty(T * w.K, dtype=torch.float32, device=dev)
    fp8_codes = torch.empty(R * H, dtype=torch.uint8, device=dev)
    fp8_scales = torch.empty(R * (H // 128), dtype=torch.float32, device=dev)
    # each layout path forced, beside the default choice (results must agree)
    paths = {n: dataclasses.replace(cfg, flags=cfg.flags | f) for n, f in LAYOUT_PATHS.items()}
    path_lay = {n: epx.Layout.empty(c, dev) for n, c in paths.items()}
    path_ws = {n: epx.workspace_for(c, dev) for n, c in paths.items()}
    extra_ops = [(n, (lambda n=n: epx.ep_dispatch_layout(paths[n], ids, path_ws[n], path_lay[n]))) for n in paths]
    # combine over NVFP4 rows: the step's own NVFP4 dispatch output stands in
    # for NVFP4 expert outputs (same format and size)
    cq_y = torch.empty(T * H, dtype=torch.bfloat16, device=dev)
    extra_ops += [("combine_bwd_probs", lambda: epx.ep_combine_bwd_probs(cfg, lay, gy, out, gprobs)),
                  ("dispatch_fp8", lambda: epx.ep_dispatch_fp8(cfg, lay, x, fp8_codes, fp8_scales)),
                  ("combine_nvfp4", lambda: epx.ep_combine_nvfp4(cfg, lay, codes, scales, rowscale, probs, cq_y))]

    def step():
        for _, fn in ops:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager_out = {k: v.clone() for k, v in (("recv", recv), ("codes", codes), ("y", y), ("gout", gout),
                                           ("gx", gx), ("token_row", lay.token_row))}

    # the whole step as one HIP graph, checked against the eager result and
    # timed beside the eager steps
    g_step = capture(torch, step)
    g_step.replay()
    torch.cuda.synchronize()
    for k, v in eager_out.items():
        cur = {"recv": recv, "codes": codes, "y": y, "gout": gout, "gx": gx, "token_row": lay.token_row}[k]
        if not torch.equal(cur.view(torch.uint8), v.view(torch.uint8)):  # bitwise: unused rows may hold NaNs
            raise RuntimeError(f"graph replay of the step changed {k}")
    log(f"[bench] warmup {args.warmup} done, graph checked; timing {args.steps} steps")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def time_steps(launch):
        """(wall ms, event ms) per step of args.steps launches, between two syncs."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(args.steps):
            launch()
        end.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, start.elapsed_time(end) / args.steps

    ms_step, gpu_ms_step = time_steps(step)          # the timed steps
    graph_ms, _ = time_steps(g_step.replay)
    for k, v in eager_out.items():
        cur = {"recv": recv, "codes": codes, "y": y, "gout": gout, "gx": gx, "token_row": lay.token_row}[k]
        if not torch.equal(cur.view(torch.uint8), v.view(torch.uint8)):
            raise RuntimeError(f"the timed steps changed {k}")

    # per-op kernel durations: a graph of LAUNCHES back-to-back launches per op,
    # bracketed by HIP events on the stream the kernels run on
    LAUNCHES, REPS, OP_WARMUP = 8, max(MIN_OP_REPS, args.steps), 5
    op_us = {}
    for n, fn in ops + extra_ops:
        def many(fn=fn):
            for _ in range(LAUNCHES):
                fn()
        g = capture(torch, many)
        for _ in range(OP_WARMUP):  # untimed: the previous op's lines leave the caches
            g.replay()
        times = []
        for _ in range(REPS):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            times.append((a, b))
        torch.cuda.synchronize()
        op_us[n] = [a.elapsed_time(b) * 1e3 / LAUNCHES for a, b in times]
        del g
    # in-step per-op durations: eager steps enqueued back to back (the queue
    # stays ahead of the GPU), an event between consecutive ops, so each op
    # runs after its predecessors as in the timed step
    IN_STEP_STEPS = max(MIN_OP_REPS // 2, 20)
    marks = []
    for _ in range(IN_STEP_STEPS):
        evs = [torch.cuda.Event(enable_timing=True)]
        evs[0].record(stream)
        for _, fn in ops:
            fn()
            evs.append(torch.cuda.Event(enable_timing=True))
            evs[-1].record(stream)
        marks.append(evs)
    torch.cuda.synchronize()
    in_step_us = {n: [m[i].elapsed_time(m[i + 1]) * 1e3 for m in marks[2:]] for i, n in enumerate(names)}
    # cold per-op durations: one launch after an untimed read of 1 GiB that
    # evicts L2 and the 256 MB MALL.  A read leaves no dirty lines behind
    # (a fill would, and the timed launch would pay for writing them back),
    # and it writes back what the previous launch left dirty.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    cold_us = {}
    for n, fn in ops + extra_ops:
        times = []
        for r in range(COLD_REPS):
            flush.sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            times.append((a, b))
        torch.cuda.synchronize()
        cold_us[n] = [a.elapsed_time(b) * 1e3 for a, b in times]
    # context: torch's own device-to-device copy of 1 GiB (read + write)
    src_c = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(1)
    copy_times = []
    for _ in range(6):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        flush.copy_(src_c)
        b.record(stream)
        copy_times.append((a, b))
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) / (statistics.median(a.elapsed_time(b) for a, b in copy_times[1:]) * 1e-3) / 1e9
    del flush, src_c

    flags = int(lay.flags.item())
    tr = lay.token_row.cpu().numpy()
    kept = int((tr >= 0).sum())
    rowoff = lay.row_offsets.cpu().numpy()
    used_rows = int(rowoff[:, -1].sum())
    seg_base = lay.seg_base.cpu().numpy()
    used = np.zeros(R, bool)  # rows past a segment's used rows are never written
    for s_ in range(w.S):
        used[seg_base[s_]:seg_base[s_] + rowoff[s_, -1]] = True
    for path, other in path_lay.items():
        for k in ("counts", "seg_base", "row_offsets", "token_row", "flags", "expert_ids", "src_info"):
            a, b = getattr(lay, k).cpu().numpy(), getattr(other, k).cpu().numpy()
            if k in ("expert_ids", "src_info"):
                a, b = a[used], b[used]
            if not np.array_equal(a, b):
                raise RuntimeError(f"the {path} layout differs from the default one in {k}")
    kept_routed = int((tr[:, :w.K] >= 0).sum())
    nbytes = algorithmic_bytes(w, kept, used_rows, kept_routed)
    def rate(n, us):
        gbps = nbytes[n] / (us * 1e-6) / 1e9
        return {"us_median": round(us, 2), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}

    per_op = {}
    trace = in_step_for(args.workload)
    for n in names + [n for n, _ in extra_ops]:
        med = statistics.median(op_us[n])
        dec = statistics.quantiles(op_us[n], n=10)
        cdec = statistics.quantiles(cold_us[n], n=10)
        gbps = nbytes[n] / (med * 1e-6) / 1e9
        per_op[n] = {"us": round(med, 2), "us_mean": round(statistics.mean(op_us[n]), 2), "us_p10": round(dec[0], 2),
                     "us_p90": round(dec[-1], 2), "reps": len(op_us[n]), "bytes": nbytes[n],
                     "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "frac_of_copy": round(gbps / copy_gbps, 4),
                     "cold": dict(rate(n, statistics.median(cold_us[n])), us_p10=round(cdec[0], 2),
                                  us_p90=round(cdec[-1], 2), reps=len(cold_us[n]))}
        if n in in_step_us:
            per_op[n]["in_step_eager"] = dict(rate(n, statistics.median(in_step_us[n])), reps=len(in_step_us[n]))
        if trace is not None and n in trace["in_step_us"]:
            per_op[n]["in_step"] = dict(rate(n, trace["in_step_us"][n]), steps=trace.get("steps"))
        log(f"[bench] {n:18s} {med:8.2f} us  {nbytes[n] / 1e6:8.2f} MB  {gbps:7.1f} GB/s  "
            f"{100 * gbps / HBM_PEAK_GBPS:5.1f}% of 8 TB/s   cold {per_op[n]['cold']['us_median']:8.2f} us "
            f"{100 * per_op[n]['cold']['frac']:5.1f}%" +
            (f"   in step {per_op[n]['in_step']['us_median']:8.2f} us {100 * per_op[n]['in_step']['frac']:5.1f}%"
             if "in_step" in per_op[n] else "") +
            (f"   eager+event {per_op[n]['in_step_eager']['us_median']:8.2f} us" if n in in_step_us else ""))
    step_bytes = sum(nbytes[n] for n in names)
    dom = max((n for n in names if n != "layout"), key=lambda n: per_op[n]["us"])
    fwd_us = per_op["layout"]["us"] + per_op["dispatch"]["us"] + per_op["combine"]["us"]
    roof = {"bound": "hbm", "kernel": dom, "achieved": per_op[dom]["GBps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": per_op[dom]["frac"], "traffic": traffic_for(dom, args.workload),
            "algorithmic_bytes_per_launch": nbytes[dom], "avg_launch_us": per_op[dom]["us"],
            "in_step_frac": per_op[dom]["in_step"]["frac"] if "in_step" in per_op[dom] else None,
            "in_step_launch_us": per_op[dom]["in_step"]["us_median"] if "in_step" in per_op[dom] else None,
            "in_step_eager_frac": per_op[dom]["in_step_eager"]["frac"],
            "cold_frac": per_op[dom]["cold"]["frac"], "cold_launch_us": per_op[dom]["cold"]["us_median"],
            "note": ("frac: median launch of graphs of 8 back-to-back launches (warm); in_step_frac: the kernel "
                     "inside the timed back-to-back steps, from the rocprofv3 trace in profiles/kernel_trace_<workload>.json "
                     "(null when the kernel sources differ from the traced ones); in_step_eager_frac: the op inside "
                     "eager steps with an event between consecutive ops, the event packet's gap included; "
                     "cold_frac: one launch after a 1 GiB read that evicts L2 and MALL")}

    result = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "gpu_ms_per_step": round(gpu_ms_step, 4),
        "graph_ms_per_step": round(graph_ms, 4),
        "launch": ("each op launched from Python through the binding, host ahead of the GPU "
                   "(graph_ms_per_step: the same step captured as one HIP graph and replayed)"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD_TITLES.get(args.workload, args.workload)}: {wl.describe(w)}",
                   "step": "layout + bf16 dispatch + NVFP4 dispatch + combine + combine_bwd + dispatch_bwd",
                   "tokens_per_step": T, "recv_rows": R, "kept_slots": kept, "used_rows": used_rows},
        "effective_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "fwd_dispatch_combine_tokens_per_s": round(T / (fwd_us * 1e-6), 1),
        "ops": per_op,
        "ops_note": ("us (median), us_mean, us_p10, us_p90, GBps, frac: warm, graphs of 8 back-to-back launches, "
                     f"{OP_WARMUP} untimed replays then {REPS} timed; in_step: the op's kernels inside the timed "
                     "steps, from the rocprofv3 kernel trace committed under profiles/ (only while the kernel "
                     "sources match it); in_step_eager: the op inside eager steps enqueued back to back "
                     f"({IN_STEP_STEPS} steps, the first 2 dropped), an event between consecutive ops, whose packet "
                     "adds a gap of about 5.6 us to each op; cold: one launch after an untimed read of 1 GiB "
                     f"that evicts L2 and MALL ({COLD_REPS} reps); frac_of_copy: against torch's 1 GiB device copy; GBps and frac use "
                     "the medians"),
        "copy_context_GBps": round(copy_gbps, 1),
        "overflow_flags": flags,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on the same batch")
        host = {"R": R, "ids": d["topk_ids"], "x": d["x"], "probs": d["probs"],
                "out": out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(R, H),
                "gy": gy.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, H),
                "grad_recv": grad_recv.view(torch.int16).cpu().numpy().view(np.uint16).reshape(R, H)}
        result["cpu_baseline"] = cpu_baseline(w, host)
        result["parity"] = parity_of_run(torch, host["oracle_results"], lay, recv, codes, scales, rowscale,
                                         y, gout, gx, R, T, H)
        log(f"[bench] parity of this run against the oracle: {result['parity']}")
    else:
        result["cpu_baseline"] = None
        result["parity"] = None
    print(json.dumps(result), flush=True)
    return 0


def parity_of_run(torch, o: dict, lay, recv, codes, scales, rowscale, y, gout, gx, R, T, H) -> dict:
    """Compare the outputs of this run's last step with the oracle's results
    on the same inputs, bit for bit (rows a layout leaves unused are not
    part of the contract and are skipped)."""
    def host(t):
        return t.contiguous().view(-1).view(torch.uint8).cpu().numpy()

    L = o["layout"]
    tr = L["token_row"]
    kept = np.unique(tr[tr >= 0])
    ok = {}
    ok["layout"] = bool(all(np.array_equal(getattr(lay, k).cpu().numpy().reshape(-1), L[k].reshape(-1))
                            for k in ("counts", "seg_base", "row_offsets", "token_row", "flags"))
                        and np.array_equal(lay.expert_ids.cpu().numpy()[kept], L["expert_ids"][kept])
                        and np.array_equal(lay.src_info.cpu().numpy()[kept], L["src_info"][kept]))
    ok["dispatch"] = bool(np.array_equal(host(recv).view(np.uint16).reshape(R, H)[kept], o["recv"][kept]))
    oc, os_, orr = o["nvfp4"]
    ok["dispatch_nvfp4"] = bool(np.array_equal(host(codes).reshape(R, H // 2)[kept], oc.reshape(R, H // 2)[kept])
                                and np.array_equal(host(scales).reshape(R, H // 16)[kept], os_.reshape(R, H // 16)[kept])
                                and np.array_equal(host(rowscale).view(np.uint16)[kept], orr.reshape(-1)[kept]))
    ok["combine"] = bool(np.array_equal(host(y).view(np.uint16).reshape(T, H), o["y"].reshape(T, H)))
    ok["combine_bwd"] = bool(np.array_equal(host(gout).view(np.uint16).reshape(R, H)[kept], o["gout"].reshape(R, H)[kept]))
    ok["dispatch_bwd"] = bool(np.array_equal(host(gx).view(np.uint16).reshape(T, H), o["gx"].reshape(T, H)))
    ok["all_bit_exact"] = all(ok.values())
    return ok


def capture(torch, fn):
    """Capture fn's launches (all on the current stream) into a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def latency_sweep(torch, epx, wl, dev, workload: str, token_counts) -> int:
    """Per-op latency (µs, graphs of 8 back-to-back launches, 3 untimed
    replays then the median of 10)
    of the workload's shape at each token count, plus the whole step (the
    ops of the benchmark step, FP8 dispatch excluded), the layout with the
    bf16, NVFP4 or FP8 dispatch made in one call, and the step with the bf16
    one in place of its two calls.  One JSON line per T."""
    # The first token count runs once more, unreported, before the others:
    # its figures came out 1-2 us high when it ran first (idle clocks, fresh
    # allocations), which 50 ms of device copies beforehand did not change.
    for i, T in enumerate([token_counts[0]] + list(token_counts)):
        w = wl.CONFIGS[workload].at_tokens(T)
        d = wl.make_workload(w)
        cfg = epx.EpConfig(num_tokens=T, hidden=w.H, num_experts=w.E, num_segments=w.S, top_k=w.K,
                           align=w.align, seg_capacity=w.capacity, shared_expert=w.shared_expert,
                           src_segment=w.src_segment)
        cfg.recv_rows = epx.ep_query(cfg).min_recv_rows
        R, H = cfg.recv_rows, w.H
        gen = torch.Generator(device=dev)
        gen.manual_seed(1)
        x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.from_numpy(d["topk_ids"].reshape(-1)).to(dev)
        probs = torch.from_numpy(d["probs"].reshape(-1)).to(dev)
        out = torch.randn(R * H, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        gy = torch.randn(T * H, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        lay, ws = epx.Layout.empty(cfg, dev), epx.workspace_for(cfg, dev)
        recv = torch.empty(R * H, dtype=torch.bfloat16, device=dev)
        codes = torch.empty(R * H // 2, dtype=torch.uint8, device=dev)
        scales = torch.empty(R * H // 16, dtype=torch.uint8, device=dev)
        rowscale = torch.empty(R, dtype=torch.bfloat16, device=dev)
        f8c = torch.empty(R * H, dtype=torch.uint8, device=dev)
        f8s = torch.empty(R * (H // 128), dtype=torch.float32, device=dev)
        y = torch.empty(T * H, dtype=torch.bfloat16, device=dev)
        gout = torch.empty(R * H, dtype=torch.bfloat16, device=dev)
        gx = torch.empty(T * H, dtype=torch.bfloat16, device=dev)
        step_ops = [("layout", lambda: epx.ep_dispatch_layout(cfg, ids, ws, lay)),
                    ("dispatch", lambda: epx.ep_dispatch(cfg, lay, x, recv)),
                    ("dispatch_nvfp4", lambda: epx.ep_dispatch_nvfp4(cfg, lay, x, codes, scales, rowscale)),
                    ("combine", lambda: epx.ep_combine(cfg, lay, out, probs, y)),
                    ("combine_bwd", lambda: epx.ep_combine_bwd(cfg, lay, gy, probs, gout)),
                    ("dispatch_bwd", lambda: epx.ep_dispatch_bwd(cfg, lay, out, gx))]
        paths = {n: dataclasses.replace(cfg, flags=cfg.flags | f) for n, f in LAYOUT_PATHS.items()}
        path_lay = {n: epx.Layout.empty(c, dev) for n, c in paths.items()}
        path_ws = {n: epx.workspace_for(c, dev) for n, c in paths.items()}
        cq_y = torch.empty(T * H, dtype=torch.bfloat16, device=dev)
        ops = step_ops + [("dispatch_fp8", lambda: epx.ep_dispatch_fp8(cfg, lay, x, f8c, f8s)),
                          ("combine_nvfp4", lambda: epx.ep_combine_nvfp4(cfg, lay, codes, scales, rowscale, probs,
                                                                         cq_y))]
        ops += [(n, (lambda n=n: epx.ep_dispatch_layout(paths[n], ids, path_ws[n], path_lay[n]))) for n in paths]
        fl_lay, fl_ws = epx.Layout.empty(cfg, dev), epx.workspace_for(cfg, dev)
        fl_recv = torch.empty(R * H, dtype=torch.bfloat16, device=dev)
        ops += [("dispatch_with_layout", lambda: epx.ep_dispatch_with_layout(cfg, ids, fl_ws, fl_lay, x, fl_recv))]
        fq = [torch.empty_like(codes), torch.empty_like(scales), torch.empty_like(rowscale)]
        ops += [("dispatch_nvfp4_with_layout",
                 lambda: epx.ep_dispatch_nvfp4_with_layout(cfg, ids, fl_ws, fl_lay, x, *fq))]
        f8q = [torch.empty_like(f8c), torch.empty_like(f8s)]
        ops += [("dispatch_fp8_with_layout", lambda: epx.ep_dispatch_fp8_with_layout(cfg, ids, fl_ws, fl_lay, x, *f8q))]
        fused_step = [("dispatch_with_layout", lambda: epx.ep_dispatch_with_layout(cfg, ids, ws, lay, x, recv))]
        fused_step += step_ops[2:]
        ops += [("step", lambda: [fn() for _, fn in step_ops])]
        ops += [("step_with_layout_dispatch", lambda: [fn() for _, fn in fused_step])]
        step_ops[0][1]()
        torch.cuda.synchronize()
        res = {}
        for n, fn in ops:
            def many(fn=fn):
                for _ in range(8):
                    fn()
            g = capture(torch, many)
            for _ in range(3):  # untimed: clocks up, the previous op's lines gone
                g.replay()
            times = []
            for _ in range(10):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                times.append((a, b))
            torch.cuda.synchronize()
            res[n] = round(statistics.median(a.elapsed_time(b) * 1e3 / 8 for a, b in times), 2)
            del g
        if i > 0:
            print(json.dumps({"latency_us": res, "workload": wl.describe(w), "tokens": T}), flush=True)
    return 0


def copy_calibration(torch, epx, dev) -> int:
    """Plain copies of known size (1 GiB read + 1 GiB written) through two
    kernels with identity routing: rocprofv3 FETCH_SIZE / WRITE_SIZE of these
    launches give the counter-to-bytes scale for each load pattern.
      - k_scatter (ep_dispatch): plain 16-byte loads of x, streaming stores;
      - k_gather (ep_dispatch_bwd, K = 1): nontemporal 16-byte loads of the
        receive rows, nontemporal stores."""
    T, H = 65536, 8192  # 65536 rows x 16 KiB = 1 GiB
    cfg = epx.EpConfig(num_tokens=T, hidden=H, num_experts=1, num_segments=1, top_k=1)
    cfg.recv_rows = epx.ep_query(cfg).min_recv_rows
    lay = epx.Layout.empty(cfg, dev)
    ws = epx.workspace_for(cfg, dev)
    ids = torch.zeros(T, dtype=torch.int32, device=dev)
    x = torch.ones(T * H, dtype=torch.bfloat16, device=dev)
    recv = torch.empty(T * H, dtype=torch.bfloat16, device=dev)
    epx.ep_dispatch_layout(cfg, ids, ws, lay)
    torch.cuda.synchronize()
    assert int((lay.token_row.cpu() == torch.arange(T, dtype=torch.int32).view(T, 1)).all()) == 1
    for _ in range(3):
        epx.ep_dispatch(cfg, lay, x, recv)
    torch.cuda.synchronize()
    for _ in range(3):
        epx.ep_dispatch_bwd(cfg, lay, recv, x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {
        "scatter": {"kernel": "k_scatter", "bytes_read": T * H * 2 + T * 4, "bytes_written": T * H * 2, "launches": 3},
        "gather": {"kernel": "k_gather", "bytes_read": T * H * 2 + T * 4, "bytes_written": T * H * 2,
                   "launches": 3}}}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
