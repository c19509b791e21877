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

