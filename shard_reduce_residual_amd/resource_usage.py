"""On-chip budget of the kernels the launch plan picks: registers, LDS, scratch and the
resulting occupancy, read from the code-object metadata of the current sources (hipcc -S of the
instantiation units; nothing is launched, no GPU is needed).

    python -m shard_reduce_residual_amd.resource_usage [--cus 256]

For each of the five workloads (and the fp8/MXFP4 variants, which share their kernel)
the plan's geometry is mapped to its kernel instantiation, whose metadata gives arch
VGPRs, AGPRs, SGPRs, spills, static LDS and private (scratch) bytes. The held-row kernel's
LDS is dynamic and follows the plan (held rows x (hidden*2 + 12 per wavefront)); path 4
(claimed rows) reserves (160 KiB - 2 KiB) / W of dynamic LDS per workgroup, which caps it
at W workgroups per CU (W = 4 for rows of less than 96 KiB of traffic, else 2). Occupancy on gfx950: a SIMD has 512 registers per lane shared by
its waves (allocated in blocks of 8), at most 8 waves per SIMD, 4 SIMDs and 160 KiB of LDS
per CU.
"""
from __future__ import annotations

import argparse
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")

REGS_PER_SIMD_LANE = 512
REG_BLOCK = 8
MAX_WAVES_PER_SIMD = 8
SIMDS_PER_CU = 4
LDS_PER_CU = 160 * 1024
TAG = {"bf16": "ActBF16", "f16": "ActF16", "f32": "PartF32"}


def _tu(pd: str, ad: str, n: int) -> str:
    lo = (n - 1) // 4 * 4 + 1
    return os.path.join(CSRC, "inst_%s_%s_n%02d_%02d.hip" % (pd, ad, lo, lo + 3))


def _metadata(src: str) -> dict:
    """Kernel metadata of one translation unit, keyed by demangled kernel name."""
    from . import build as b

    with tempfile.TemporaryDirectory() as tmp:
        asm = os.path.join(tmp, "k.s")
        cmd = [b.HIPCC] + [f for f in b.FLAGS if f != "-fPIC"] + [
            "--cuda-device-only", "-S", src, "-o", asm]
        subprocess.run(cmd, check=True, capture_output=True)
        text = open(asm).read()
    meta = text[text.index("amdhsa.kernels:"):]
    out = {}
    for blk in re.split(r"\n  - ", meta):
        m = re.search(r"\.name:\s+(\S+)", blk)
        if not m:
            continue
        name = subprocess.run(["c++filt", m.group(1)], capture_output=True,
                              text=True).stdout.strip()

        def field(k):
            f = re.search(r"\.%s:\s+(\d+)" % k, blk)
            return int(f.group(1)) if f else 0
        out[name] = {k: field(k) for k in ("vgpr_count", "agpr_count", "sgpr_count",
                                           "vgpr_spill_count", "sgpr_spill_count",
                                           "group_segment_fixed_size",
                                           "private_segment_fixed_size")}
    return out


def occupancy(regs_total: int, waves_per_wg: int, lds_per_wg: int) -> dict:
    """Waves per SIMD and workgroups per CU for a kernel on gfx950."""
    alloc = -(-max(regs_total, 1) // REG_BLOCK) * REG_BLOCK
    waves_simd = min(MAX_WAVES_PER_SIMD, REGS_PER_SIMD_LANE // alloc)
    wg_by_regs = waves_simd * SIMDS_PER_CU // waves_per_wg
    wg_by_lds = LDS_PER_CU // lds_per_wg if lds_per_wg else 1 << 30
    wgs = min(wg_by_regs, wg_by_lds)
    return {"reg_alloc": alloc, "workgroups_per_cu": wgs,
            "waves_per_simd": wgs * waves_per_wg // SIMDS_PER_CU,
            "limited_by": "LDS" if wg_by_lds < wg_by_regs else "registers"}


def report(cus: int = 256) -> str:
    sys.path.insert(0, ROOT)
    import workloads

    import shard_reduce_residual_amd as arf

    lines = ["| workload | plan | kernel | arch VGPR | AGPR | total regs | SGPR | spills (V/S) "
             "| LDS per workgroup | scratch | workgroups per CU | waves per SIMD | limited by |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    cache = {}
    for key in ("c0", "c1", "c2", "c3", "c4"):
        w = workloads.WORKLOADS[key]
        pd = {"bf16": 0, "f16": 1, "f32": 2}[w.partial_dtype]
        quant = {None: arf.ARF_QUANT_NONE, "per_tensor": arf.ARF_QUANT_PER_TENSOR,
                 "per_token": arf.ARF_QUANT_PER_TOKEN}[w.quant]
        plan = arf.arf_get_plan_quant(w.n_shards, w.tokens, w.hidden, pd, quant, cus)
        tu = _tu(w.partial_dtype, w.act_dtype, w.n_shards)
        if tu not in cache:
            cache[tu] = _metadata(tu)
        pt, at = "arf::" + TAG[w.partial_dtype], "arf::" + TAG[w.act_dtype]
        if plan["path"] == 3:
            # held calls without a quantised copy take the QUANT = false form
            name = "void arf::fused_held_rows<%s, %s, %d, %d, %d, %s>(arf::Params)" % (
                pt, at, w.n_shards, plan["chunks"], plan["waves"],
                "true" if w.quant else "false")
            rows = -(-w.tokens // plan["grid"])
            dyn = rows * (2 * w.hidden + 12 * plan["waves"])
        else:
            cand = [n for n in cache[tu] if n.startswith(
                "void arf::fused_reduce_add_rmsnorm<%s, %s, %d, %d, %d, %s," % (
                    pt, at, w.n_shards, plan["chunks"],
                    plan["waves"], "true" if plan["path"] == 1 else "false"))]
            assert len(cand) == 1, cand
            name = cand[0]
            row_bytes = w.n_shards * w.hidden * w.sp + 6 * w.hidden
            per_cu = 4 if row_bytes < 96 * 1024 else 2
            dyn = (LDS_PER_CU - 2048) // per_cu if plan["path"] == 4 else 0
        m = cache[tu][name]
        regs = m["vgpr_count"]            # on gfx950: arch VGPRs + AGPRs, as allocated
        agpr = m["agpr_count"]
        lds = m["group_segment_fixed_size"] + dyn
        occ = occupancy(regs, plan["waves"], lds)
        lines.append("| %s | path %d, %d waves x %d chunks, grid %d | `%s` | %d | %d | %d | %d "
                     "| %d / %d | %d B | %d B | %d | %d | %s |" % (
                         w.name, plan["path"], plan["waves"], plan["chunks"], plan["grid"],
                         name.replace("void ", "").replace("(arf::Params)", ""), regs - agpr, agpr,
                         regs, m["sgpr_count"], m["vgpr_spill_count"], m["sgpr_spill_count"],
                         lds, m["private_segment_fixed_size"], occ["workgroups_per_cu"],
                         occ["waves_per_simd"], occ["limited_by"]))
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--cus", type=int, default=256)
    print(report(ap.parse_args().cus))


if __name__ == "__main__":
    main()
