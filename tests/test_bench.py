# Host-side behaviour of bench.py that needs no GPU: the one-GPU contract,
# the HBM traffic record's keying to the kernel source, and the quantiles.
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

HEADLINE = "llama3.1-8b_down_wgrad_4096x14336x32768"


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_resolves_for_the_committed_kernel():
    got, note = bench.measured_traffic(HEADLINE)
    assert got is not None, note
    assert "FETCH_SIZE" in note and "WRITE_SIZE" in note
    # The record is per launch of the main kernel: far above the kernel's
    # algorithmic bytes (operands once, output once), far below 1 TB.
    assert 0.4e9 < got < 1e12


def _record(summary):
    with open(summary) as f:
        for ln in f:
            if ln.startswith("traffic-record: "):
                return json.loads(ln[len("traffic-record: "):])
    raise AssertionError("no traffic record")


@pytest.mark.parametrize("change", ["sha", "workload"])
def test_traffic_record_is_dropped_when_it_no_longer_applies(tmp_path, change):
    rec = _record(bench.TRAFFIC_SUMMARY)
    if change == "sha":
        rec["source_sha256"] = "0" * 64
    else:
        rec["workload"] = "another_workload"
    p = tmp_path / "summary.md"
    p.write_text("traffic-record: " + json.dumps(rec) + "\n")
    got, note = bench.measured_traffic(HEADLINE, summary=str(p))
    assert got is None
    assert ("changed" in note) if change == "sha" else ("another workload" in note)


def test_missing_summary_gives_no_traffic(tmp_path):
    got, note = bench.measured_traffic(HEADLINE, summary=str(tmp_path / "absent.md"))
    assert got is None and note


def test_quantiles_of_a_known_sample():
    q = bench.quantiles([float(i) for i in range(1, 101)])
    assert q == {"median": 50.5, "p10": 10.9, "p90": 90.1}


def test_headline_workload_is_a_bench_workload():
    wl = bench.workloads()
    w, call = wl["l8b_down_wgrad"]
    assert w.name == HEADLINE and call == 0
    for bs in (1, 2, 4, 8, 16):
        for op in ("fwd", "dgrad", "wgrad"):
            assert f"l8b_oproj_bs{bs}_{op}" in wl
