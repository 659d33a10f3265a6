"""bench.py's host-side logic that needs no GPU: more than one GPU is refused
with a message (the benchmark runs on one GPU), and the HBM-traffic figure of
the roofline is taken from the committed counter summary only while the kernel
sources still match it."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_code_only_ignores_comments_and_blank_runs():
    bench = _bench()
    a = "int f(int x) {  // the answer\n  return x + 1; /* one */\n}\n"
    b = "int f(int x) {\n\n  return x + 1;\n}  // changed comment\n"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(a.replace("x + 1", "x + 2"))


def test_traffic_record_is_used_only_while_the_sources_match(tmp_path, monkeypatch):
    """`roofline.traffic` comes from the committed counter summary only while the
    kernel sources still hash to the recorded value; otherwise it is null."""
    bench = _bench()
    sha = bench.kernel_hash("linear")
    f = tmp_path / "traffic.md"
    rec = {"linear:720p_81f": {"source_sha": sha, "bytes_per_launch": 123}}
    f.write_text("x\n```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("linear", "720p_81f") == 123
    assert bench.traffic_for("linear", "480p_81f") is None       # no record for that workload
    rec["linear:720p_81f"]["source_sha"] = "0" * 16
    f.write_text("```json\n" + json.dumps(rec) + "\n```\n")
    assert bench.traffic_for("linear", "720p_81f") is None       # stale record
    f.write_text("no json block here")
    assert bench.traffic_for("linear", "720p_81f") is None
