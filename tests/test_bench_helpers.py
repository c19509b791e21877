"""Host-side helpers of bench.py (no GPU): the kernel-source digest that ties
the committed rocprofv3 figures to the code they were taken on, and the
readers that report those figures only while it matches."""

import json
import os
import shutil

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources and profiles, with bench.ROOT pointing at it."""
    for p in bench.KERNEL_SOURCES:
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), dst)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_digest_ignores_comments_and_whitespace(tree):
    d0 = bench.source_digest()
    p = tree / bench.KERNEL_SOURCES[0]
    text = p.read_text()
    p.write_text("// a new comment line\n/* and a block\n   comment */\n" + text.replace("\n", "\n\n"))
    assert bench.source_digest() == d0
    p.write_text(text + "\nstatic int extra_code_line;\n")
    assert bench.source_digest() != d0


def test_profile_readers_follow_the_digest(tree):
    d = bench.source_digest()
    trace = {"workload": "dsv3", "source_digest": d, "steps": 3,
             "in_step_us": {"dispatch": 90.0}, "step_span_us": 400.0}
    traffic = {"workload": "dsv3", "source_digest": d, "ops": {"dispatch": {"bytes_per_launch": 123}}}
    (tree / "profiles" / "kernel_trace_dsv3.json").write_text(json.dumps(trace))
    (tree / "profiles" / "traffic_dsv3.json").write_text(json.dumps(traffic))
    assert bench.in_step_for("dsv3")["in_step_us"]["dispatch"] == 90.0
    assert bench.traffic_for("dispatch", "dsv3") == 123
    assert bench.traffic_for("combine", "dsv3") is None          # op not measured
    assert bench.in_step_for("skewed") is None                     # no file for that workload
    p = tree / bench.KERNEL_SOURCES[-1]
    p.write_text(p.read_text() + "\nstatic int changed_kernel_code;\n")
    assert bench.in_step_for("dsv3") is None                       # kernels changed since the trace
    assert bench.traffic_for("dispatch", "dsv3") is None



def test_profile_summarizer_maps_kernels_to_ops():
    """bench_profiles.py attributes each traced kernel to the bench op it
    serves (the rank kernel's second template argument is its path)."""
    import bench_profiles as bp

    assert bp.short("void epx::(anonymous namespace)::k_scatter<false, true>(epx::MoveArgs)") == "k_scatter<false, true>"
    cases = {"k_scatter<false, true>": "dispatch", "k_scatter<true, true>": "combine_bwd",
             "k_gather<true, true>": "combine", "k_gather<false, true>": "dispatch_bwd",
             "k_layout_hist<2>": "layout_hist", "k_layout_rank<2, 1, false, 256>": "layout_rank",
             "k_layout_rank<1, 3, false, 256>": "layout_count", "k_layout_rank<1, 2, false, 2048>": "layout_small",
             "k_layout_sp<4, 256, true>": "layout_lookback", "k_layout_sp<4, 256, false>": "layout_barrier",
             "k_nvfp4_wg<1>": "dispatch_nvfp4", "k_fp8_wg<8, false>": "dispatch_fp8",
             "k_combine_nvfp4<true>": "combine_nvfp4", "k_probs_grad": "combine_bwd_probs",
             "k_layout_chunks": None}
    for k, op in cases.items():
        assert bp.op_of(k) == op, k
    assert bp.pattern_of("k_gather<true, true>") == "gather" and bp.pattern_of("k_scatter<false, true>") == "scatter"


def test_profile_summarizer_step_timeline(tmp_path, monkeypatch):
    """bench_profiles.py takes the in-step durations from the steps whose
    kernels run back to back (the timed eager steps and the graph replays),
    leaves out the eager steps with an event between ops, and reports the
    idle time between consecutive back-to-back steps."""
    import csv

    import bench_profiles as bp

    names = ["void epx::(anonymous namespace)::k_layout_hist<2>(epx::LayoutArgs)",
             "void epx::(anonymous namespace)::k_layout_rank<2, 1, false, 256>(epx::LayoutArgs)",
             "void epx::(anonymous namespace)::k_scatter<false, true>(epx::MoveArgs)",
             "void epx::(anonymous namespace)::k_nvfp4_wg<1>(epx::Nvfp4Args)",
             "void epx::(anonymous namespace)::k_gather<true, true>(epx::MoveArgs)",
             "void epx::(anonymous namespace)::k_scatter<true, true>(epx::MoveArgs)",
             "void epx::(anonymous namespace)::k_gather<false, true>(epx::MoveArgs)"]
    dur_ns = [4000, 7000, 90000, 29000, 91000, 90000, 89000]
    rows, t = [], 1_000_000

    def step(gap_between_ops, gap_after):
        nonlocal t
        for n, d in zip(names, dur_ns):
            rows.append({"Kernel_Name": n, "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d + gap_between_ops
        t += gap_after - gap_between_ops

    for _ in range(3):
        step(0, 0)            # eager timed steps: back to back
    for _ in range(3):
        step(0, 8000)         # graph replays: 8 us between steps
    for _ in range(2):
        step(5600, 20000)     # eager steps with an event before every op
    d = tmp_path / "run" / "p_trace_dsv3"
    d.mkdir(parents=True)
    with open(d / "dsv3_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bp, "OUT", str(tmp_path / "run"))
    monkeypatch.setattr(bp, "RUN", "run")
    monkeypatch.setattr(bp, "PROF", str(tmp_path / "profiles"))
    avg, in_step, whole = bp.trace_summary("dsv3")
    assert in_step["dispatch"] == 90.0 and in_step["combine"] == 91.0 and in_step["layout_rank"] == 7.0
    assert whole == sum(dur_ns) / 1e3
    doc = json.loads((tmp_path / "profiles" / "kernel_trace_dsv3.json").read_text())
    assert doc["steps"] == 6 and doc["eager_event_gap_us"] == 5.6
    assert doc["in_step_us"]["layout"] == 11.0
    md = (tmp_path / "profiles" / "kernel_trace_dsv3.md").read_text()
    assert "3 graph-replay boundaries" not in md  # boundaries are counted between consecutive steps
    assert "2 graph-replay boundaries, median 8.00 us" in md and "eager step boundaries, median 0.00 us" in md
