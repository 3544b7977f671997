"""Host-side pieces of bench.py: the multi-GPU refusal and the traffic
bookkeeping (counters keyed to the kernels' code, comments excluded)."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(root, name, text):
    d = os.path.join(root, "streaming_attention_amd", "csrc")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, name), "w", encoding="utf-8") as f:
        f.write(text)


def test_code_hash_ignores_comments_and_blank_lines_only(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write(tmp_path, "k.hip", "int f(int x) {\n  return x + 1;\n}\n")
    h0 = bench.code_hash(["k.hip"])
    _write(tmp_path, "k.hip", "// a note\nint f(int x) {   // inline\n\n  return x + 1;\n}\n")
    assert bench.code_hash(["k.hip"]) == h0
    _write(tmp_path, "k.hip", "int f(int x) {\n  return x + 2;\n}\n")
    assert bench.code_hash(["k.hip"]) != h0


def test_measured_traffic_is_null_once_the_code_changes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write(tmp_path, "k.hip", "int f();\n")
    entry = {"sources": ["k.hip"], "sha256_16": bench.code_hash(["k.hip"]), "fetch_kib": 10, "write_kib": 3}
    monkeypatch.setitem(bench.TRAFFIC, "t", entry)
    assert bench.measured_traffic("t") == int(10 * 1024 / bench.FETCH_SCALE + 3 * 1024 / bench.WRITE_SCALE)
    _write(tmp_path, "k.hip", "int g();\n")
    assert bench.measured_traffic("t") is None


def test_every_traffic_entry_names_existing_sources():
    for name, t in bench.TRAFFIC.items():
        for f in t["sources"]:
            assert os.path.exists(os.path.join(ROOT, "streaming_attention_amd", "csrc", f)), (name, f)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr
