"""bench.py's contract where no GPU is needed: it refuses more than one GPU
before touching torch, and it reports the committed HBM-traffic figure only
while the GEMM source is the one the counters were taken on (its hash
ignores comments and blank space, not code)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, timeout=120, env=env, cwd=ROOT)


def test_refuses_more_than_one_gpu():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""            # no JSON line


def test_refuses_a_distributed_launch():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_code_hash_ignores_comments_not_code(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("/* header */\nint f(int x) {\n\n  return x + 1;    // another comment\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.code_hash(str(a)) == bench.code_hash(str(b))
    assert bench.code_hash(str(a)) != bench.code_hash(str(c))


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    src = tmp_path / "long_context_anti_amd" / "csrc" / "gemm_bf16.hip"
    src.parent.mkdir(parents=True)
    src.write_text("__global__ void k() {}\n")
    prof = tmp_path / "profiles" / "llama1b_rmt_L16_S128_gateup_hbm_traffic.md"
    prof.parent.mkdir()
    prof.write_text(f"gemm_bf16.hip code sha256 prefix: {bench.code_hash(str(src))} (comments and blank space "
                    "removed)\n\ntraffic (bench roofline field) = 1.500 GB + 0.250 GB = 1.750 GB per launch.\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() == 1_750_000_000
    src.write_text("// a comment changes nothing\n__global__ void k() {}\n")
    assert bench.measured_traffic() == 1_750_000_000
    src.write_text("__global__ void k() { }\n__global__ void k2() {}\n")
    assert bench.measured_traffic() is None
    prof.unlink()
    assert bench.measured_traffic() is None
