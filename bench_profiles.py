"""Summaries of rocprofv3 runs of bench.py, written to profiles/.

    python bench_profiles.py RUN_DIR [workload ...]

RUN_DIR (a path relative to the repository root) holds what the commands
listed in each summary wrote, run from the repository root:

  * RUN_DIR/bench_<workload>.log: `python bench.py [--workload W]
    --no-cpu-baseline` (its JSON line gives each op's algorithmic bytes);
  * RUN_DIR/p_trace_<workload>/: the rocprofv3 kernel trace of bench.py;
  * RUN_DIR/p_fetch_<workload>/, RUN_DIR/p_write_<workload>/: FETCH_SIZE
    (with GRBM_GUI_ACTIVE) and WRITE_SIZE counter passes;
  * RUN_DIR/p_cfetch/, RUN_DIR/p_cwrite/: the same counters on
    `bench.py --copy-calibration` (the counter-to-bytes scale);
  * RUN_DIR/p_lds/, RUN_DIR/p_atom/ (optional): LDS and atomic counters.

For each workload it writes profiles/kernel_trace_<workload>.{md,json} and
profiles/traffic_<workload>.{md,json} (and profiles/lds_atomics_dsv3.md),
stamped with the kernel-source digest; bench.py reports the in-step
durations and the counter traffic from the JSON files only while that
digest matches the sources.
"""
import collections
import csv
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

RUN = None  # RUN_DIR as given on the command line (it appears in the commands quoted)
OUT = None  # the same, as a path
PROF = os.path.join(ROOT, "profiles")
WORKLOADS = ["dsv3", "skewed", "capacity", "nvfp4"]
TITLES = {"dsv3": "DeepSeek-V3-shaped share (T=4096, H=7168, E=256/8, K=8, A=128)",
          "skewed": "skewed routing (T=8192, H=4096, E=128/8, K=8, A=128, Zipf 1.2)",
          "capacity": "capacity overflow (T=16384, H=2048, E=64/4, K=6, C=27 036, Zipf 1.5)",
          "nvfp4": "NVFP4 dispatch with a fused shared expert (T=4096, H=7168, E=256/8, K=8+1, A=128)"}
# load pattern of each kernel, for the counter scale: plain 16-byte loads
# (scatter copy) or nontemporal loads (gather copy)
NT_LOAD_KERNELS = ("k_gather", "k_probs_grad")


def op_of(k):
    """op of a short kernel name, e.g. 'k_scatter<false, true>' -> 'dispatch'."""
    m = re.match(r"(\w+)(?:<(.*)>)?$", k)
    if not m:
        return None
    name, targs = m.group(1), [x.strip() for x in (m.group(2) or "").split(",")]
    if name == "k_layout_hist":
        return "layout_hist"
    if name == "k_layout_rank":
        return {"1": "layout_rank", "2": "layout_small", "3": "layout_count"}[targs[1]]
    if name == "k_layout_sp":
        return "layout_lookback" if targs[2] == "true" else "layout_barrier"
    if name == "k_scatter":
        return "combine_bwd" if targs[0] == "true" else "dispatch"
    if name == "k_gather":
        return "combine" if targs[0] == "true" else "dispatch_bwd"
    return {"k_nvfp4": "dispatch_nvfp4", "k_nvfp4_wg": "dispatch_nvfp4", "k_fp8": "dispatch_fp8",
            "k_fp8_wg": "dispatch_fp8", "k_probs_grad": "combine_bwd_probs",
            "k_combine_nvfp4": "combine_nvfp4"}.get(name)


# kernels of each bench op (the layout ops share kernels: their trace rows
# cover every layout launch of the run)
OP_KERNEL_OPS = {"layout": ["layout_hist", "layout_rank"], "layout_two_kernel": ["layout_hist", "layout_rank"],
                 "layout_count": ["layout_count"], "layout_lookback": ["layout_lookback"],
                 "layout_barrier": ["layout_barrier"]}
STEP_OPS = ["layout_hist", "layout_rank", "dispatch", "dispatch_nvfp4", "combine", "combine_bwd", "dispatch_bwd"]
STEP_LABELS = ["layout (histogram)", "layout (rank)", "dispatch", "dispatch_nvfp4", "combine", "combine_bwd",
               "dispatch_bwd"]


def short(name):
    n = name
    if n.startswith("void "):
        n = n[5:]
    n = n.replace("epx::(anonymous namespace)::", "")
    if "(" in n:
        n = n[:n.index("(")]
    return n


def csv_rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def counters(path):
    """{short kernel: {counter: [per-dispatch values]}}"""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for r in csv_rows(path):
        per[short(r["Kernel_Name"])][r["Counter_Name"]][int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    return {k: {c: list(d.values()) for c, d in v.items()} for k, v in per.items()}


def bench_line(log):
    with open(log) as f:
        lines = [ln for ln in f if ln.startswith("{")]
    return json.loads(lines[-1])


def wflag(wk):
    return "" if wk == "dsv3" else f" --workload {wk}"


def trace_summary(wk):
    d = os.path.join(OUT, f"p_trace_{wk}")
    cmd = (f"rocprofv3 --kernel-trace --stats -f csv -d {RUN}/p_trace_{wk} -o {wk} -- "
           f"python3 bench.py{wflag(wk)} --steps 20 --warmup 2 --no-cpu-baseline")
    tr = sorted(csv_rows(os.path.join(d, f"{wk}_kernel_trace.csv")), key=lambda r: int(r["Start_Timestamp"]))
    tr = [(short(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in tr]
    tr = [(n, a, b) for n, a, b in tr if op_of(n)]
    dur = collections.defaultdict(list)
    for n, a, b in tr:
        dur[n].append((b - a) / 1e3)
    ops = [op_of(n) for n, _, _ in tr]
    steps = [tr[i:i + len(STEP_OPS)] for i in range(len(tr) - len(STEP_OPS) + 1)
             if ops[i:i + len(STEP_OPS)] == STEP_OPS]
    L = [f"# Kernel trace: {TITLES[wk]}", "",
         "Command (from the repository root on an MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "",
         "    " + cmd, "",
         f"Summarized from its CSV output with `python bench_profiles.py {RUN}`.", "",
         "Each op runs 8x back-to-back inside a HIP graph per timing replay (at least 50 timed replays), plus the "
         "timed steps (eager, then as graph replays), eager steps with events and one launch per op after a cache "
         "flush; the table averages every launch of the kernel in the run, so the layout kernels' rows also hold "
         "the forced-path layout launches that use them.", "",
         "| kernel | op | calls | avg us | median us | min us | max us |", "|---|---|---|---|---|---|---|"]
    for n in sorted(dur, key=lambda n: -statistics.mean(dur[n])):
        x = dur[n]
        L.append(f"| `{n}` | {op_of(n)} | {len(x)} | {statistics.mean(x):.2f} | {statistics.median(x):.2f} | "
                 f"{min(x):.2f} | {max(x):.2f} |")
    # the timed steps (eager and graph-replayed) run their kernels back to
    # back; the eager steps of the bench's event timing have an event
    # between consecutive ops
    gaps = [[(st[j + 1][1] - st[j][2]) / 1e3 for j in range(len(STEP_OPS) - 1)] for st in steps]
    graph = [st for st, g in zip(steps, gaps) if max(g) < 1.0]
    eager_gaps = [x for g in gaps if max(g) >= 1.0 for x in g[1:] if x < 100.0]
    # idle time between consecutive back-to-back steps: the graph replays
    # pay the graph launch, the eager ones follow each other directly
    between = [(b[0][1] - a[-1][2]) / 1e3 for a, b in zip(graph, graph[1:]) if b[0][1] - a[-1][2] < 50_000]
    L += ["", f"In-step durations: the step's kernels inside the {len(graph)} back-to-back steps of the same run "
          "(the timed steps of bench.py: eager launches, then graph replays; no gap between the kernels of a step). "
          "Inputs are cold there, and each kernel also pays for write-backs its predecessors left.", "",
          "| op | kernel | median us | min us | max us |", "|---|---|---|---|---|"]
    in_step = {}
    for j, label in enumerate(STEP_LABELS):
        x = [(st[j][2] - st[j][1]) / 1e3 for st in graph]
        in_step[STEP_OPS[j]] = statistics.median(x)
        L.append(f"| {label} | `{graph[0][j][0]}` | {statistics.median(x):.2f} | {min(x):.2f} | {max(x):.2f} |")
    whole = [(st[-1][2] - st[0][1]) / 1e3 for st in graph]
    L.append(f"| whole step (first kernel start to last kernel end) | | {statistics.median(whole):.2f} | "
             f"{min(whole):.2f} | {max(whole):.2f} |")
    if between:
        small = [x for x in between if x < 3.0]
        large = [x for x in between if x >= 3.0]
        L += ["", "Idle time from one step's last kernel end to the next step's first kernel start: "
              + (f"{len(small)} eager step boundaries, median {statistics.median(small):.2f} us" if small else "no eager boundaries")
              + "; " + (f"{len(large)} graph-replay boundaries, median {statistics.median(large):.2f} us"
                        if large else "no graph-replay boundaries") + "."]
    if eager_gaps:
        L += ["", f"The bench's eager steps with an event between consecutive ops ({len(steps) - len(graph)} steps in "
              f"this run) show a median gap of {statistics.median(eager_gaps):.2f} us between one op's last kernel "
              "and the next op's first: the event packet. bench.py's in_step_eager figures include it."]
    doc = {"workload": wk, "source_digest": bench.source_digest(), "command": cmd, "steps": len(graph),
           "in_step_us": {"layout": statistics.median([(st[1][2] - st[0][1]) / 1e3 for st in graph]),
                          **{op: round(v, 3) for op, v in in_step.items() if not op.startswith("layout_")}},
           "step_span_us": round(statistics.median(whole), 3),
           "eager_event_gap_us": round(statistics.median(eager_gaps), 3) if eager_gaps else None}
    doc["in_step_us"]["layout"] = round(doc["in_step_us"]["layout"], 3)
    with open(os.path.join(PROF, f"kernel_trace_{wk}.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    with open(os.path.join(PROF, f"kernel_trace_{wk}.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    avg = collections.defaultdict(float)
    for n, x in dur.items():
        avg[op_of(n)] += statistics.mean(x)
    return avg, in_step, statistics.median(whole)


def calibration():
    """Counter scale per load pattern from the two 1 GiB copies."""
    fe = counters(os.path.join(OUT, "p_cfetch", "copy_counter_collection.csv"))
    wr = counters(os.path.join(OUT, "p_cwrite", "copy_counter_collection.csv"))
    T, H = 65536, 8192
    true_r, true_w = (T * H * 2 + T * 4) / 1024, T * H * 2 / 1024
    out = {}
    for pat, prefix in (("scatter", "k_scatter<"), ("gather", "k_gather<")):
        k = next(k for k in fe if k.startswith(prefix))
        fk, wk = statistics.mean(fe[k]["FETCH_SIZE"]), statistics.mean(wr[k]["WRITE_SIZE"])
        out[pat] = {"kernel": k, "true_read_KiB": true_r, "true_write_KiB": true_w, "FETCH_SIZE_KiB": fk,
                    "WRITE_SIZE_KiB": wk, "fetch_factor": round(true_r / fk, 4), "write_factor": round(true_w / wk, 4),
                    "launches": len(fe[k]["FETCH_SIZE"])}
    return out


def pattern_of(kernel):
    return "gather" if kernel.startswith(NT_LOAD_KERNELS) else "scatter"


def traffic_summary(wk, alg, avg_us, calib):
    fe = counters(os.path.join(OUT, f"p_fetch_{wk}", f"{wk}_counter_collection.csv"))
    wr = counters(os.path.join(OUT, f"p_write_{wk}", f"{wk}_counter_collection.csv"))
    cmds = [f"rocprofv3 --pmc FETCH_SIZE GRBM_GUI_ACTIVE -f csv -d {RUN}/p_fetch_{wk} -o {wk} -- python3 "
            f"bench.py{wflag(wk)} --steps 2 --warmup 1 --no-cpu-baseline",
            f"rocprofv3 --pmc WRITE_SIZE -f csv -d {RUN}/p_write_{wk} -o {wk} -- python3 bench.py{wflag(wk)} "
            "--steps 2 --warmup 1 --no-cpu-baseline"]
    ccmds = [f"rocprofv3 --pmc FETCH_SIZE -f csv -d {RUN}/p_cfetch -o copy -- python3 bench.py --copy-calibration",
             f"rocprofv3 --pmc WRITE_SIZE -f csv -d {RUN}/p_cwrite -o copy -- python3 bench.py --copy-calibration"]
    doc = {"workload": wk, "source_digest": bench.source_digest(),
           "calibration": dict(calib, commands=ccmds,
                               note="bytes = FETCH_SIZE KiB * 1024 * fetch_factor + WRITE_SIZE KiB * 1024 * "
                                    "write_factor, with the factors of the copy whose loads the kernel's loads "
                                    "resemble: gather (nontemporal loads) for k_gather and k_probs_grad, scatter "
                                    "(plain loads) for the others"),
           "commands": cmds, "ops": {}}
    order = ["dispatch", "dispatch_nvfp4", "combine", "combine_bwd", "dispatch_bwd", "combine_bwd_probs",
             "dispatch_fp8", "combine_nvfp4", "layout", "layout_count", "layout_lookback", "layout_barrier"]
    rows = []
    for op in order:
        if op not in alg:
            continue
        ks = [k for k in fe if op_of(k) in OP_KERNEL_OPS.get(op, [op])]
        if not ks:
            continue
        fk = sum(statistics.mean(fe[k]["FETCH_SIZE"]) for k in ks)
        wk_ = sum(statistics.mean(wr[k]["WRITE_SIZE"]) for k in ks)
        gui = sum(statistics.mean(fe[k]["GRBM_GUI_ACTIVE"]) for k in ks)
        by = int(round(sum(statistics.mean(fe[k]["FETCH_SIZE"]) * 1024 * calib[pattern_of(k)]["fetch_factor"] +
                           statistics.mean(wr[k]["WRITE_SIZE"]) * 1024 * calib[pattern_of(k)]["write_factor"]
                           for k in ks)))
        us = sum(avg_us.get(o, 0.0) for o in OP_KERNEL_OPS.get(op, [op]))
        doc["ops"][op] = {"kernels": ks, "pattern": sorted({pattern_of(k) for k in ks}), "FETCH_SIZE_KiB": fk,
                          "WRITE_SIZE_KiB": wk_, "GRBM_GUI_ACTIVE": gui, "bytes_per_launch": by,
                          "algorithmic_bytes": alg[op], "launches": len(fe[ks[0]]["FETCH_SIZE"]),
                          "trace_avg_us": round(us, 2)}
        prec = 2 if op.startswith("layout") else 1
        rows.append(f"| {op} | {', '.join(sorted({pattern_of(k) for k in ks}))} | {fk:.0f} | {wk_:.0f} | "
                    f"{by / 1e6:.{prec}f} | {alg[op] / 1e6:.{prec}f} | {by / alg[op]:.3f} | {gui:.0f} | {gui / 8 / 2400:.2f} | "
                    f"{us:.2f} |")
    with open(os.path.join(PROF, f"traffic_{wk}.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    L = [f"# HBM traffic per launch: {TITLES[wk]}", "",
         "Counters (one pass each, from the repository root on an MI355X):", ""]
    L += ["    " + x for x in cmds]
    L += ["", f"Summarized from their CSV output with `python bench_profiles.py {RUN}`."]
    L += ["", "Scale: the same counters on two plain copies of known size (1 GiB read + 1 GiB written, identity "
          "routing): through the dispatch scatter (plain 16-byte loads) and through the dispatch-backward gather "
          "(nontemporal 16-byte loads):", ""]
    L += ["    " + x for x in ccmds]
    L += [""]
    for pat, c in calib.items():
        L.append(f"- {pat} copy (`{c['kernel']}`): FETCH_SIZE {c['FETCH_SIZE_KiB']:.0f} KiB for "
                 f"{c['true_read_KiB']:.0f} KiB read (factor {c['fetch_factor']:.4f}); WRITE_SIZE "
                 f"{c['WRITE_SIZE_KiB']:.0f} KiB for {c['true_write_KiB']:.0f} KiB written (factor "
                 f"{c['write_factor']:.4f}).")
    L += ["", "Each kernel's counters take the factors of the copy with its load pattern (gather: k_gather, "
          "k_probs_grad; scatter: every other kernel). GRBM_GUI_ACTIVE: GPU-busy cycles per launch in the FETCH "
          "pass, summed over the 8 XCDs; divided by 8 and by the 2.4 GHz peak clock it gives the launch's busy "
          "time in that pass, next to the kernel trace's average of the timing run.", "",
          "| op | pattern | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic MB (scaled) | algorithmic MB | "
          "traffic / algorithmic | GRBM_GUI_ACTIVE | busy us (/ 8 XCDs / 2.4 GHz) | kernel-trace avg us |",
          "|---|---|---|---|---|---|---|---|---|---|"] + rows
    L += ["", f"Kernel sources digest: `{doc['source_digest']}` (bench.py reports this traffic only while the "
          "digest matches)."]
    with open(os.path.join(PROF, f"traffic_{wk}.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    return doc


def lds_summary():
    lds = counters(os.path.join(OUT, "p_lds", "dsv3_counter_collection.csv"))
    atm = counters(os.path.join(OUT, "p_atom", "dsv3_counter_collection.csv"))
    L = ["# LDS and atomic counters: DeepSeek-V3-shaped share", "",
         "Commands (one pass each, from the repository root on an MI355X):", "",
         "    rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_LDS_ADDR_CONFLICT SQ_WAVES "
         f"SQ_INSTS_VALU -f csv -d {RUN}/p_lds -o dsv3 -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
         "    rocprofv3 --pmc TCC_ATOMIC TCC_EA0_ATOMIC TCP_TCC_ATOMIC_WITH_RET_REQ TCP_TCC_ATOMIC_WITHOUT_RET_REQ "
         f"-f csv -d {RUN}/p_atom -o dsv3 -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline", "",
         f"Summarized from their CSV output with `python bench_profiles.py {RUN}`.", "",
         "Per launch, averaged over the launches of the run. SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE are in "
         "cycles summed over the chip; the conflict share is their ratio.", "",
         "| kernel | op | waves | VALU instr | LDS instr | LDS bank-conflict cycles | LDS active cycles | "
         "conflict share | LDS addr-conflict | TCC atomics | TCC->EA atomics | TCP atomics w/ ret | "
         "TCP atomics w/o ret |",
         "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted((k for k in lds if op_of(k)), key=lambda k: (op_of(k), k)):
        def m(src, c):
            return statistics.mean(src[k][c]) if k in src and c in src[k] else float("nan")
        bc, ia = m(lds, "SQ_LDS_BANK_CONFLICT"), m(lds, "SQ_LDS_IDX_ACTIVE")
        share = f"{bc / ia:.3f}" if ia else "n/a"
        L.append(f"| `{k}` | {op_of(k)} | {m(lds, 'SQ_WAVES'):.0f} | {m(lds, 'SQ_INSTS_VALU'):.0f} | "
                 f"{m(lds, 'SQ_INSTS_LDS'):.0f} | {bc:.0f} | {ia:.0f} | {share} | {m(lds, 'SQ_LDS_ADDR_CONFLICT'):.0f} | "
                 f"{m(atm, 'TCC_ATOMIC'):.0f} | {m(atm, 'TCC_EA0_ATOMIC'):.0f} | "
                 f"{m(atm, 'TCP_TCC_ATOMIC_WITH_RET_REQ'):.0f} | {m(atm, 'TCP_TCC_ATOMIC_WITHOUT_RET_REQ'):.0f} |")
    with open(os.path.join(PROF, "lds_atomics_dsv3.md"), "w") as f:
        f.write("\n".join(L) + "\n")


def main():
    global RUN, OUT
    if len(sys.argv) < 2:
        print(__doc__, file=sys.stderr)
        return 2
    RUN = sys.argv[1].rstrip("/")
    OUT = os.path.join(ROOT, RUN)
    wks = sys.argv[2:] or [w for w in WORKLOADS if os.path.isdir(os.path.join(OUT, f"p_trace_{w}"))]
    calib = calibration()
    for wk in wks:
        avg, in_step, whole = trace_summary(wk)
        alg = {op: v["bytes"] for op, v in bench_line(os.path.join(OUT, f"bench_{wk}.log"))["ops"].items()}
        doc = traffic_summary(wk, alg, avg, calib)
        print(wk, "step", round(whole, 2), "in-step", {k: round(v, 2) for k, v in in_step.items()},
              "traffic/alg", {k: round(v["bytes_per_launch"] / v["algorithmic_bytes"], 3)
                              for k, v in doc["ops"].items()})
    if os.path.isdir(os.path.join(OUT, "p_lds")):
        lds_summary()
    print("digest", bench.source_digest(), "calibration",
          {p: (c["fetch_factor"], c["write_factor"]) for p, c in calib.items()})


if __name__ == "__main__":
    sys.exit(main())
