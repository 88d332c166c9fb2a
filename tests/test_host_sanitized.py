"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host/abi_host_checks.cpp is built with vsa_api.cpp (sanitizers on the
host code only; the kernel launchers are stubs that report a failed launch)
and run on the CPU: validation of every field, workspace and saved-buffer
carving, the host list checker and the latent helper. No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not installed")
def test_abi_host_logic_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host_checks")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-x", "hip", *san, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "block_sparse_video_cube_amd", "csrc", "vsa_api.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_host_checks.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host checks passed" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
