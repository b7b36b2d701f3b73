"""Host logic of bench.py (no GPU): the one-GPU refusal, the roofline
fields, and the rule that a committed HBM-traffic figure is reported only
while the kernel sources it was measured on are unchanged."""
import hashlib
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

TAG = "rowop_glu_selectinfer_decode"
SOURCES = ["rowop_b1.hip", "sffn_device.h"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_roofline_fields():
    rf = bench.roofline("k", 8_000_000, 2.0, traffic=8_100_000)
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] == pytest.approx(4000.0)
    assert rf["frac"] == pytest.approx(0.5)
    assert rf["traffic"] == 8_100_000


def _sha(csrc, sources=SOURCES):
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


@pytest.mark.parametrize("tag", [TAG, "rowop_glu_swiglu_top50_layer", "rowop_relu_gate_moe",
                                 "tiered_down_spax", "tiered_qkv_spax", "axpy_b1_swiglu_top50_layer",
                                 "moe_gathered_layer", "union_down_b1", "union_down_b4",
                                 "union_down_b8", "union_down_b16"])
def test_committed_traffic_follows_its_sources(tag):
    with open(os.path.join(ROOT, "profiles", f"traffic_{tag}.json")) as fh:
        rec = json.load(fh)
    sources = rec.get("sources", SOURCES)
    got = bench.measured_traffic(tag, sources)
    if rec["source_sha256"] == _sha(bench.CSRC, sources):
        assert got == rec["bytes_per_launch"] and got > 0
    else:
        assert got is None


def test_traffic_dropped_when_a_source_changes(tmp_path, monkeypatch):
    root, csrc = tmp_path / "root", tmp_path / "csrc"
    (root / "profiles").mkdir(parents=True)
    csrc.mkdir()
    for name in SOURCES:
        shutil.copy(os.path.join(bench.CSRC, name), csrc / name)
    rec = {"source_sha256": _sha(str(csrc)), "bytes_per_launch": 12345}
    (root / "profiles" / f"traffic_{TAG}.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    assert bench.measured_traffic(TAG, SOURCES) == 12345
    with open(csrc / SOURCES[0], "a") as fh:
        fh.write("\n// edited\n")
    assert bench.measured_traffic(TAG, SOURCES) is None
    assert bench.measured_traffic("no_such_kernel", SOURCES) is None


def test_cpu_baseline_reports_all_cores_and_one():
    calls = []
    cb = bench.cpu_baseline(lambda i: calls.append(i), 0.01, "item(s) of nothing", per_unit=2)
    assert cb["kind"] == "oracle" and cb["unit"] == "us/token" and cb["cores"] >= 1
    assert cb["value"] > 0 and cb["sample"].endswith("item(s) of nothing")
    assert cb["one_core"]["cores"] == 1 and cb["one_core"]["value"] > 0
    assert calls[0] == 0


def test_default_workload_is_the_full_run():
    import argparse
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert a.workload == "all" and a.gpus == 1
    assert isinstance(a, argparse.Namespace) and a.cpu_seconds_sub > 0
