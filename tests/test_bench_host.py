"""Host-side checks of bench.py that need no GPU: the counter records in
profiles/ are reported only while every source they were taken from is
unchanged, and the one-GPU contract."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_sha1_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1; // one\n}\n")
    b.write_text("/* header */ int f(int x) {   return x + 1;\n}  // other\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.code_sha1(str(a)) == bench.code_sha1(str(b))
    assert bench.code_sha1(str(a)) != bench.code_sha1(str(c))


def test_counter_record_follows_its_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    (tmp_path / "profiles").mkdir()
    rec = {"sources": {"k.hip": bench.code_sha1(str(src))}, "kernels": {"k": {"hbm_bytes": 7}}}
    (tmp_path / "profiles" / "r.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._counter_record("r") == rec
    src.write_text("__global__ void k() {}  // a comment changes nothing\n")
    assert bench._counter_record("r") == rec
    src.write_text("__global__ void k() { int x = 1; }\n")
    assert bench._counter_record("r") is None
    assert bench._counter_record("missing") is None


@pytest.mark.parametrize("name", ["traffic_long_1m", "mfma_long_1m", "traffic_decode_256"])
def test_committed_records_name_existing_sources(name):
    rec = json.load(open(os.path.join(ROOT, "profiles", name + ".json")))
    assert rec["sources"] and rec["kernels"]
    for path in rec["sources"]:
        assert os.path.isfile(os.path.join(ROOT, path)), path


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
