"""Build libarfuse.so for gfx950 with hipcc (in-tree, parallel per translation unit)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "arfuse")
LIB = os.path.join(HERE, "libarfuse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 add/mul/fma; the
# remaining options are ordinary release flags.
FLAGS = ["-O3", "--offload-arch=" + ARCH, "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"   # host pass: unknown target feature, harmless
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every csrc/*.hip and link shard_reduce_residual_amd/libarfuse.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    # export the C ABI (arf_*) only: the kernels' launchers and host stubs stay local, so
    # the library cannot clash with another one that instantiates the same templates
    vmap = os.path.join(OBJDIR, "exports.map")
    with open(vmap, "w") as f:
        f.write("{\n  global: arf_*;\n  local: *;\n};\n")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--version-script=" + vmap,
           "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
