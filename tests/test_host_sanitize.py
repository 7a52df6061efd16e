"""The metadata builders under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/host/meta_sanitize.cpp`` drives cp_meta_build,
cp_allgather_meta_build and cp_allgather_packed_meta_build with seeded random
arguments (valid and invalid) into exactly sized heap buffers and checks the
bounds of every table the kernels index.  The builders are host-only C++, so
they are compiled here with g++ (no GPU code involved)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_metadata_builders_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "meta_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "host", "meta_sanitize.cpp"),
           os.path.join(ROOT, "context_prefill_attention_amd", "csrc", "cp_meta.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe), "30000"], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "ok: 30000 cases, 0 failures" in run.stdout
    # every builder saw accepted and rejected arguments
    for line in run.stdout.splitlines():
        if line.startswith("builder"):
            ok = int(line.split("ok ")[1].split()[0])
            invalid = int(line.split("invalid ")[1].split()[0])
            assert ok > 1000 and invalid > 100, line
