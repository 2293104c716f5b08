"""Host-side logic of bench.py (CPU): the roofline byte counts, the decode
record, the counter-record lookup keyed by the kernel source's hash, and the
one-GPU guard."""
import glob
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,per_weight", [("dsv3_bf16", 2.0), ("dsv3_fp8", 1.0), ("dsv3_fp4", 0.5 + 1.0 / 32)])
def test_weight_bytes_per_expert(name, per_weight):
    # gate, up and down: 3 H I weights; fp4 packs two per byte plus one UE8M0
    # scale byte per 32 weights
    s = synthetic.spec(name)
    assert bench.weight_bytes_per_expert(s) == pytest.approx(3 * s.H * s.I * per_weight)


def test_decode_record_counts_touched_experts_once():
    s = synthetic.spec("qwen_decode", T=64)
    counts = np.zeros(s.E, dtype=np.int64)
    counts[:59] = 4
    m = {"counts": counts, "ms_per_step": 0.25, "n_stages": 5.0}
    rec = bench.decode_record(s, m, 200)
    alg = 59 * 3 * s.H * s.I * 2
    assert rec["touched_experts"] == 59 and rec["alg_bytes"] == alg
    assert rec["achieved_GBs"] == pytest.approx(alg / 0.25e-3 / 1e9, abs=0.05)   # (rounded to 0.1 GB/s)
    assert rec["frac"] == pytest.approx(rec["achieved_GBs"] / bench.PEAK_HBM_GBS, abs=1e-4)


def test_recorded_traffic_matches_the_committed_records():
    recs = glob.glob(os.path.join(ROOT, "profiles", "*.traffic.json"))
    assert recs, "no counter records under profiles/"
    for path in recs:
        r = json.load(open(path))
        src = os.path.join(ROOT, r["source"])
        fresh = hashlib.sha256(open(src, "rb").read()).hexdigest() == r["source_sha256"]
        got = bench.recorded_traffic(r["workload"], r["kernel"])
        if fresh:
            assert got == pytest.approx(r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"])
        else:
            assert got is None
    assert bench.recorded_traffic("dsv3_bf16", "no_such_kernel") is None


def test_recorded_traffic_is_dropped_when_the_source_changes(tmp_path, monkeypatch):
    # a record whose source hash no longer matches gives no traffic
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text("// kernel v2\n")
    rec = {"workload": "w", "kernel": "k<0>", "source": "k.hip",
           "source_sha256": hashlib.sha256(b"// kernel v1\n").hexdigest(),
           "fetch_bytes_per_launch": 10.0, "write_bytes_per_launch": 5.0}
    (tmp_path / "profiles" / "k.w.traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("w", "k<0>") is None
    rec["source_sha256"] = hashlib.sha256(b"// kernel v2\n").hexdigest()
    (tmp_path / "profiles" / "k.w.traffic.json").write_text(json.dumps(rec))
    assert bench.recorded_traffic("w", "k<0>") == 15.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
