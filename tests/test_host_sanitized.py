"""libarfuse's host-side dispatcher (argument validation, launch plan, geometry override)
under AddressSanitizer and UndefinedBehaviorSanitizer, CPU only. The dispatcher source is
built for the host with the sanitizers (its device code as usual), against stub kernel
tables, and tests/host_sanitize_driver.hip drives every entry point; any sanitizer report
or a failed check fails."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "shard_reduce_residual_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_dispatcher_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitized")
    cmd = [HIPCC, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "arfuse_host.hip"), os.path.join(HERE, "host_sanitize_driver.hip"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    # the HIP runtime is not instrumented and keeps allocations until exit: no leak check
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
