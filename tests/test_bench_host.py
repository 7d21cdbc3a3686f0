"""Host-side logic of bench.py (no GPU): the one-GPU contract and the rule
that the reported HBM traffic belongs to the kernel source it was measured on."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def _record(path):
    kv = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_traffic_record_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    kv = _record(bench.TRAFFIC_FILE)
    src = os.path.join(ROOT, kv["kernel_source"])
    current = hashlib.sha256(open(src, "rb").read()).hexdigest()
    expect = float(kv["traffic_bytes_per_launch"]) if current == kv["kernel_source_sha256"] else None
    assert bench.measured_traffic(True) == expect
    assert bench.measured_traffic(False) is None          # another workload: never reported
    # a record taken on another version of the kernel is not reported
    stale = tmp_path / "stale.txt"
    stale.write_text(open(bench.TRAFFIC_FILE).read().replace(kv["kernel_source_sha256"], "0" * 64))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic(True) is None


def test_traffic_record_is_consistent():
    kv = _record(bench.TRAFFIC_FILE)
    copy_kib = int(kv["copy_bytes"]) / 1024
    fs = copy_kib / float(kv["copy_fetch_kib"])     # the scales, from the copy's counts
    ws = copy_kib / float(kv["copy_write_kib"])
    assert abs(float(kv["fetch_scale"]) - fs) < 1e-3 and abs(float(kv["write_scale"]) - ws) < 1e-3
    fetch = float(kv["fetch_kib_per_dispatch"]) * fs * 1024
    write = float(kv["write_kib_per_dispatch"]) * ws * 1024
    assert abs(fetch + write - float(kv["traffic_bytes_per_launch"])) <= 1e-6 * (fetch + write)


def test_sampled_oracle_baseline_scales_to_the_whole_call():
    """The sampled baseline times evenly spaced units and scales by the
    fraction sampled; when the whole call fits the budget it is repeated."""
    seen = []

    def run(units):   # a stand-in workload: 10 ms per unit
        seen.append(list(units))
        import time
        time.sleep(0.01 * len(units))

    r = bench.cpu_baseline_sampled(run, list(range(1000)), 0.1, lambda t: 1.0 / t, "calls/s",
                                   "units")
    assert seen[0] == [500]                            # calibration: the middle unit
    n = len(seen[1])
    assert 5 <= n <= 20 and seen[1] == sorted(set(seen[1]))
    assert 0.05 < r["value"] <= 0.101                   # whole call ~ 1000 x 10 ms (sleep never short)
    assert r["kind"] == "oracle" and f"{n} of 1000 units" in r["sample"]
    seen.clear()
    r = bench.cpu_baseline_sampled(run, [0, 1], 0.2, lambda t: t, "s", "units")
    assert all(s == [0, 1] for s in seen[1:]) and len(seen) >= 3
    assert "the whole call (2 units)" in r["sample"] and 0.0199 <= r["value"] < 0.04
