"""bench.py's reporting logic that needs no GPU: the measured HBM traffic is
reported only for the kernel source and build flags it was measured with."""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_committed_traffic_matches_current_sources():
    prof = os.path.join(ROOT, "profiles")
    fwd = bench._measured_traffic(os.path.join(prof, "traffic.json"), "sta_forward.hip", "720p", "bytes_per_launch")
    bwd = bench._measured_traffic(os.path.join(prof, "traffic_bwd.json"), "sta_backward.hip", "720p",
                                  "bytes_per_call")
    assert fwd is not None and fwd > 3.54e9       # at least the algorithmic bytes
    assert bwd is not None and bwd > 0


def test_traffic_is_null_for_another_source_flags_or_workload(tmp_path):
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    cases = {
        "hash": dict(t, kernel_source_sha256="0" * 64),
        "flags": dict(t, kernel_build_flags=t["kernel_build_flags"][:-1]),
        "noflags": {k: v for k, v in t.items() if k != "kernel_build_flags"},
    }
    for name, doc in cases.items():
        p = tmp_path / f"{name}.json"
        p.write_text(json.dumps(doc))
        assert bench._measured_traffic(str(p), "sta_forward.hip", "720p", "bytes_per_launch") is None, name
    p = tmp_path / "same.json"
    p.write_text(json.dumps(t))
    assert bench._measured_traffic(str(p), "sta_forward.hip", "720p", "bytes_per_launch") == t["bytes_per_launch"]
    assert bench._measured_traffic(str(p), "sta_forward.hip", "long", "bytes_per_launch") is None
    assert bench._measured_traffic(str(tmp_path / "missing.json"), "sta_forward.hip", "720p", "bytes") is None


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
