"""AddressSanitizer / UndefinedBehaviorSanitizer runs on the CPU (no GPU needed):

- the oracle, compiled into tests/sanitize/oracle_checks.c, runs every entry point on a small
  seeded case and rejects bad arguments;
- the library's host side (the C ABI's argument checks, workspace sizing and layout queries in
  csrc/api.hip and csrc/probe.hip), built with the sanitizers on its host code and linked against
  launchers that abort if reached, refuses every bad call before any device work.

Sanitizers apply to host code only (the device code is built as usual)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "lora_mixture_experts_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-fno-sanitize-recover=undefined", "-fopenmp", os.path.join(SAN, "oracle_checks.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_abi_host_checks_under_asan_ubsan(tmp_path):
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *host_san]
    objs = []
    for src in (os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "probe.hip"),
                os.path.join(SAN, "stub_launchers.hip")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_host_checks.o")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "abi_host_checks.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", "-fno-gpu-sanitize", *objs, drv,
          "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout
