"""Host-side checks of bench.py: the one-GPU contract and the use of committed counter
summaries (no GPU needed)."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits_with_message(argv, env):
    e = dict(os.environ, **env)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def _write_summary(root, workload, src_hash, nbytes):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"traffic_gate_up_{workload}.txt"), "w") as f:
        f.write(f"workload: {workload}\nkernel_source_hash: {src_hash}\n"
                f"fetch_scale: 2.0\nwrite_scale: 1.0\nhbm_bytes_per_launch: {nbytes}\n")


def test_traffic_read_only_for_the_same_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abcdef0123456789")
    assert bench.measured_traffic("decode") is None  # no summary
    _write_summary(str(tmp_path), "decode", "abcdef0123456789", 2956944967.5)
    assert bench.measured_traffic("decode") == pytest.approx(2956944967.5)
    _write_summary(str(tmp_path), "decode", "0000000000000000", 2956944967.5)
    assert bench.measured_traffic("decode") is None  # taken on other kernel sources
    assert bench.measured_traffic("fg") is None


def test_kernel_source_hash_covers_the_kernel_sources():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    csrc = os.path.join(ROOT, "lora_mixture_experts_amd", "csrc")
    assert any(f.endswith(".hip") for f in os.listdir(csrc))
