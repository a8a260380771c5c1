"""Host-side contract of bench.py (no GPU): the one-GPU guard and the lookup
of committed HBM-traffic counters, which must go null as soon as the kernel
sources differ from the ones the counters were taken on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_refused():
    # exits before importing torch or touching a device
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=60, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_kernel_source_sha_tracks_sources():
    sha = bench.kernel_source_sha()
    assert len(sha) == 16 and int(sha, 16) >= 0
    assert bench.kernel_source_sha() == sha          # deterministic


def test_kernel_source_sha_sees_code_not_comments(tmp_path):
    src = tmp_path / "csrc"
    src.mkdir()
    f = src / "k.hip"
    f.write_text('int a = 1;  // one\n/* block\n comment */\nconst char* s = "// kept";\n')
    base = bench.kernel_source_sha(str(src))
    f.write_text('int a = 1;  // the value one\n\n/* another\n block comment */\nconst char* s = "// kept";\n')
    assert bench.kernel_source_sha(str(src)) == base
    f.write_text('int a = 2;  // one\n/* block\n comment */\nconst char* s = "// kept";\n')
    assert bench.kernel_source_sha(str(src)) != base
    f.write_text('int a = 1;  // one\n/* block\n comment */\nconst char* s = "// kEpt";\n')
    assert bench.kernel_source_sha(str(src)) != base
    assert bench.code_text('x = "a\\"b"; // c') == 'x = "a\\"b";'
    (src / "quant_kernels.hip").write_text("int q = 1;\n")       # not a GEMM source
    f.write_text('int a = 1;  // one\n/* block\n comment */\nconst char* s = "// kept";\n')
    with_q = bench.kernel_source_sha(str(src))
    (src / "quant_kernels.hip").write_text("int q = 2;\n")
    assert bench.kernel_source_sha(str(src)) == with_q == base


def _with_traffic(tmp_path, monkeypatch, record):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(record))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))


def test_traffic_reported_for_matching_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    _with_traffic(tmp_path, monkeypatch, {"kernel_source_sha": sha,
                                          "workloads": {"prefill_norm": {"traffic_bytes": 123456}}})
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    assert bench.measured_traffic("prefill_norm") == 123456
    assert bench.measured_traffic("decode") is None         # no counters for it


def test_traffic_null_once_sources_change(tmp_path, monkeypatch):
    _with_traffic(tmp_path, monkeypatch, {"kernel_source_sha": "0000000000000000",
                                          "workloads": {"prefill_norm": {"traffic_bytes": 123456}}})
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "ffffffffffffffff")
    assert bench.measured_traffic("prefill_norm") is None


def test_traffic_null_without_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("prefill_norm") is None


def test_committed_counters_name_their_sources():
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert len(t["kernel_source_sha"]) == 16
    for w, rec in t["workloads"].items():
        assert rec["traffic_bytes"] > 0, w
        assert "gemm" in rec["kernel"], w
