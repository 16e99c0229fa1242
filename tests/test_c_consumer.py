"""libarfuse used from plain C: tests/c_abi_consumer.c includes only include/arfuse.h (and
the HIP runtime's C API for its buffers), links -larfuse, and checks its results against
the oracle's C library. The CPU test builds it here with -Werror and runs the argument
checks; the GPU test runs the copy that build() made in-tree on device buffers from
hipMalloc, with no Python or PyTorch in the process."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import __graft_entry__ as entry  # noqa: E402


def test_c_consumer_builds_and_checks_arguments(tmp_path):
    exe = str(tmp_path / "c_abi_consumer")
    b = subprocess.run(entry.c_consumer_command(exe), capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe, "cpu"], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok cpu"), r.stdout + r.stderr


@pytest.mark.gpu
def test_c_consumer_on_the_gpu():
    exe = entry.C_CONSUMER
    assert os.path.exists(exe), "tests/c_abi_consumer is missing: run __graft_entry__.build()"
    r = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok gpu"), r.stdout[-4000:] + r.stderr[-4000:]
    assert r.stdout.count("case ") == 5, r.stdout


def test_header_is_strict_c(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "arfuse.h"\nint main(void) { return arf_version() == ARF_VERSION ? 0 : 1; }\n')
    for std in ("c89", "c99", "c11"):
        r = subprocess.run(["gcc", "-std=" + std, "-pedantic", "-Wall", "-Wextra", "-Werror",
                            "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)],
                           capture_output=True, text=True, timeout=60)
        assert r.returncode == 0, (std, r.stderr)
