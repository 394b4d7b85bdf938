"""bench.py's host-side contract, checked without a GPU: the one-GPU guard,
the kernel-source hash the traffic counters are tied to, and the traffic
value it reports only while that hash matches."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_sha_covers_the_gemm_sources():
    b = _bench()
    sha = b.kernel_sha()
    assert len(sha) == 16 and int(sha, 16) >= 0
    assert any(p.endswith("k_gemm6.hip") for p in b.GEMM_SOURCES)
    assert any(p.endswith("sqf_device.h") for p in b.GEMM_SOURCES)


def test_traffic_only_for_the_profiled_kernel(tmp_path, monkeypatch):
    b = _bench()
    f = tmp_path / "traffic.txt"
    f.write_text(f"# comment = ignored\nkernel_sha = {b.kernel_sha()}\nhbm_bytes_per_launch = 123456\n")
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(f))
    assert b.read_traffic() == 123456.0
    f.write_text("kernel_sha = 0000000000000000\nhbm_bytes_per_launch = 123456\n")
    assert b.read_traffic() is None
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert b.read_traffic() is None
