#!/usr/bin/env python3
"""Benchmark of the fused reduce + residual + RMSNorm (+fp8) epilogue on one MI355X.

A step is one launch of the whole fused path (rank-order sum of N shard partials,
residual add and store, RMSNorm and store, fp8 copy with per-token scales) over one
batch of seeded synthetic input already resident in HBM. The default workload is the
largest one: N=8 shards, 8192 tokens, hidden 16384, bf16, per-token fp8 (3.09 GB of
algorithmic traffic per step).

Prints ONE JSON line. ``value`` is algorithmic GB/s from the wall clock around the K
timed steps; ``roofline.achieved`` uses the fused kernel's average duration from HIP
events recorded on the stream it is launched on. ``cpu_baseline`` times the oracle on
a bounded sample of the same workload on the host's cores.
"""
import argparse
import hashlib
import glob
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused reduce+residual+RMSNorm GB/s & tokens/s; fraction of HBM peak"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def source_digest() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "shard_reduce_residual_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "fused_%s_counters.txt" % workload_name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_digest") != source_digest() or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


class Runner:
    """Inputs and outputs of one workload on the GPU (``sets`` rotating copies) and the
    launch of the fused path on ``stream``."""

    def __init__(self, w, dev, stream, sets=1):
        import torch

        import workloads

        self.w, self.stream = w, stream
        t, h = w.tokens, w.hidden
        adt = workloads.TORCH_DTYPES[w.act_dtype]
        self.sets = []
        for _ in range(sets):
            p, r, g = workloads.generate(w, dev)
            rout = torch.empty((t, h), dtype=adt, device=dev)
            nout = torch.empty((t, h), dtype=adt, device=dev)
            q = torch.empty((t, h), dtype=torch.uint8, device=dev) if w.quant else None
            sc_out = (torch.empty((t,), dtype=torch.float32, device=dev)
                      if w.quant == "per_token" else None)
            # any positive per-tensor scale runs the same instructions
            sc_in = (torch.tensor([0.01], dtype=torch.float32, device=dev)
                     if w.quant == "per_tensor" else None)
            self.sets.append((p, r, g, rout, nout, q, sc_out, sc_in))
        self.k = 0
        # the inputs are generated on the current stream; launches go to ``stream``
        torch.cuda.synchronize()

    def step(self):
        import shard_reduce_residual_amd as arf

        w = self.w
        p, r, g, rout, nout, q, sc_out, sc_in = self.sets[self.k % len(self.sets)]
        self.k += 1
        if w.quant is None:
            arf.arf_reduce_add_rmsnorm(p, r, g, w.eps, residual_out=rout, norm_out=nout,
                                       stream=self.stream)
        else:
            mode = (arf.ARF_QUANT_PER_TOKEN if w.quant == "per_token"
                    else arf.ARF_QUANT_PER_TENSOR)
            arf.arf_reduce_add_rmsnorm_quant(p, r, g, w.eps, q, mode, scale_in=sc_in,
                                             scale_out=sc_out, residual_out=rout,
                                             norm_out=nout, stream=self.stream)

    def measure(self, steps, warmup):
        """(wall ms per step, kernel ms per launch from events on the launch stream)."""
        import torch

        torch.cuda.synchronize()
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(self.stream)
        for _ in range(steps):
            self.step()
        ev1.record(self.stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps

    def distribution(self, launches, flush=None):
        """Per-launch durations (ms, sorted) from an event pair around each launch on the
        launch stream. ``flush()``, if given, runs before each pair, outside it."""
        import torch

        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(launches)]
        for e0, e1 in ev:
            if flush is not None:
                flush()
            e0.record(self.stream)
            self.step()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) for e0, e1 in ev)


def plan_of(w):
    """The launch plan of the workload's call (its quantised copy included)."""
    import shard_reduce_residual_amd as arf

    quant = {None: arf.ARF_QUANT_NONE, "per_tensor": arf.ARF_QUANT_PER_TENSOR,
             "per_token": arf.ARF_QUANT_PER_TOKEN}[w.quant]
    return arf.arf_get_plan_quant(w.n_shards, w.tokens, w.hidden,
                                  {"bf16": 0, "f16": 1, "f32": 2}[w.partial_dtype], quant)


def percentiles_us(ms_sorted):
    """median, p10 and p90 (µs) of sorted per-launch durations in ms."""
    def at(q):
        return ms_sorted[min(len(ms_sorted) - 1, int(round(q * (len(ms_sorted) - 1))))] * 1e3
    return {"median": round(at(0.5), 3), "p10": round(at(0.1), 3), "p90": round(at(0.9), 3),
            "launches": len(ms_sorted)}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4", help="c0..c4 (default c4)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target oracle time for the CPU baseline (0: skip it)")
    ap.add_argument("--no-copy-probe", action="store_true",
                    help="skip the HBM probes (read, write, copy, workload mix)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the accumulation and token-slice variants")
    ap.add_argument("--secondary", default="c3",
                    help="second workload reported in the 'secondary' object ('' for none)")
    ap.add_argument("--profile-variant", default=None,
                    choices=["fused", "mxfp4", "acc_partial", "reduce_rows", "epilogue",
                             "copy"],
                    help="launch only this variant of the workload (warmup + steps times) "
                         "and print its timing, for profiler runs; no contract line")
    ap.add_argument("--survey", action="store_true",
                    help="time the planned path on a grid of shapes against the serial "
                         "read-then-write probe for the same bytes; one JSON line per "
                         "shape, no contract line")
    return ap.parse_args()


# Shapes of the survey: (shards, tokens, hidden, partial type, quantised copy). Shapes
# whose partials exceed 2 GiB are left out.
SURVEY_SHAPES = (
    [(n, t, h, "bf16", None) for n in (2, 4, 8, 16) for h in (2048, 4096, 8192, 16384)
     for t in (1024, 4096, 16384)]
    + [(4, t, h, "f32", None) for h in (4096, 7168, 8192) for t in (2048, 8192)]
    + [(8, 4096, 8192, "bf16", "per_token"), (8, 8192, 16384, "bf16", "per_token"),
       (8, 4096, 4096, "bf16", "per_token"), (4, 16384, 4096, "bf16", "per_token")]
    + [(4, 2048, 7168, "bf16", "per_tensor"), (8, 2048, 7168, "bf16", "per_tensor"),
       (2, 1024, 8192, "bf16", "per_tensor"), (4, 2048, 7168, "f32", "per_tensor")])


def survey(args, dev, stream):
    """The plan on every shape of SURVEY_SHAPES (bf16 activations, synthetic inputs of
    c4's distribution): kernel time from events over ``steps`` launches rotating input
    sets of at least 1.5 GB, and the serial pass of direction_probes for the same bytes."""
    import dataclasses

    import torch

    import shard_reduce_residual_amd as arf
    import workloads

    base = workloads.WORKLOADS["c4"]
    for n, t, h, pdt, quant in SURVEY_SHAPES:
        sp = 4 if pdt == "f32" else 2
        if n * t * h * sp > 2 ** 31:
            continue
        w = dataclasses.replace(base, name="survey", n_shards=n, tokens=t, hidden=h,
                                partial_dtype=pdt, quant=quant)
        B = w.algorithmic_bytes()
        run = Runner(w, dev, stream, sets=max(1, min(6, -(-1_500_000_000 // B))))
        plan = plan_of(w)
        _, kms = run.measure(args.steps, args.warmup)
        d = direction_probes(w, [s[0] for s in run.sets], stream, reps=8)
        gbs = B / (kms * 1e-3) / 1e9
        print(json.dumps({"shards": n, "tokens": t, "hidden": h, "partials": pdt,
                          "quant": quant, "plan": plan, "kernel_us": round(kms * 1e3, 2),
                          "GBs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                          "serial_us": d["serial_us"],
                          "frac_of_serial": round(d["serial_us"] / (kms * 1e3), 4)}),
              flush=True)
        del run
        torch.cuda.empty_cache()
    return 0


def profile_variant(args, w, run, stream):
    """One variant of the workload on its own, for rocprofv3 runs: the fused call as
    timed (fused), the MXFP4 copy in place of the fp8 one (mxfp4), accumulation in the
    partial type (acc_partial), one rank's token slice of the reduce (reduce_rows), the
    epilogue over gathered reduced values (epilogue), or the library's streaming copy of
    exactly 1 GiB (copy: the calibration of the HBM byte counters)."""
    import torch

    import shard_reduce_residual_amd as arf

    p, r, g, rout, nout, q, sc_out, sc_in = run.sets[0]
    t, h, n = w.tokens, w.hidden, w.n_shards
    mode = arf.ARF_QUANT_PER_TOKEN if w.quant == "per_token" else arf.ARF_QUANT_PER_TENSOR
    quant = dict(quant_out=q, mode=mode, scale_in=sc_in, scale_out=sc_out) if w.quant else {}
    v = args.profile_variant
    if v == "copy":
        one_gib = 1 << 30
        src = torch.empty(one_gib, dtype=torch.uint8, device=rout.device)
        dst = torch.empty(one_gib, dtype=torch.uint8, device=rout.device)

        def fn():
            arf.arf_stream_copy(dst, src, one_gib, stream=stream)
        nbytes = 2 * one_gib
    elif v == "fused":
        fn, nbytes = run.step, w.algorithmic_bytes()
    elif v == "acc_partial":
        def fn():
            arf.arf_fused_epilogue(p, r, g, w.eps, residual_out=rout, norm_out=nout,
                                   accumulate=arf.ARF_ACC_PARTIAL, stream=stream, **quant)
        nbytes = w.algorithmic_bytes()
    elif v == "mxfp4":
        q4 = torch.empty((t, h // 2), dtype=torch.uint8, device=rout.device)
        s4 = torch.empty((t, h // 32), dtype=torch.uint8, device=rout.device)

        def fn():
            arf.arf_fused_epilogue(p, r, g, w.eps, residual_out=rout, norm_out=nout,
                                   quant_out=q4, mode=arf.ARF_QUANT_MXFP4, scale_out=s4,
                                   stream=stream)
        nbytes = (w.with_tokens(t).algorithmic_bytes()
                  - (t * h + 4 * t if w.quant == "per_token" else (t * h + 4 if w.quant else 0))
                  + t * h // 2 + t * h // 32)
    else:
        sums = torch.empty((t, h), dtype=rout.dtype, device=rout.device)
        arf.arf_reduce_rows(p, sums, stream=stream)
        cnt = t // n + (1 if t % n else 0)
        if v == "reduce_rows":
            def fn():
                arf.arf_reduce_rows(p, sums, row_begin=0, row_count=cnt, stream=stream)
            nbytes = n * cnt * h * w.sp + cnt * h * w.sa
        else:
            def fn():
                if w.quant:
                    arf.arf_reduce_add_rmsnorm_quant(sums.view(1, t, h), r, g, w.eps, q, mode,
                                                     scale_in=sc_in, scale_out=sc_out,
                                                     residual_out=rout, norm_out=nout,
                                                     stream=stream)
                else:
                    arf.arf_reduce_add_rmsnorm(sums.view(1, t, h), r, g, w.eps,
                                               residual_out=rout, norm_out=nout, stream=stream)
            nbytes = w.algorithmic_bytes() - n * t * h * w.sp + t * h * w.sa
    ms = _events_ms(fn, stream, args.steps, args.warmup)
    print(json.dumps({"variant": v, "workload": w.name, "launches": args.steps,
                      "kernel_ms": round(ms, 5), "algorithmic_bytes": nbytes,
                      "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 2)}), flush=True)
    return 0


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the fused epilogue on one GPU; it has "
              "no multi-GPU mode (asked for --gpus %d, WORLD_SIZE %d)"
              % (args.gpus, world), file=sys.stderr)
        return 2

    import torch

    import shard_reduce_residual_amd as arf
    import workloads

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    if args.survey:
        return survey(args, dev, stream)
    t, h = w.tokens, w.hidden
    B = w.algorithmic_bytes()
    # workloads smaller than 1.5 GB rotate input/output sets so that the 256 MB Infinity
    # Cache cannot serve a launch (c0-c2 still fit in it: see decode_cold for those)
    run = Runner(w, dev, stream, sets=max(1, min(8, -(-1_500_000_000 // B))))
    if args.profile_variant:
        return profile_variant(args, w, run, stream)
    ms_per_step, kernel_ms = run.measure(args.steps, args.warmup)
    value = B / (ms_per_step * 1e-3) / 1e9
    achieved = B / (kernel_ms * 1e-3) / 1e9
    traffic = read_traffic(w.name)
    launch_us = percentiles_us(run.distribution(max(args.steps, 20)))
    sus = sustained(run, kernel_ms, B)
    p, r, g, rout, nout, q, sc_out, sc_in = run.sets[0]

    secondary = None
    if args.secondary:
        w2 = workloads.WORKLOADS[args.secondary]
        B2 = w2.algorithmic_bytes()
        # rotate enough buffer sets that the 256 MB Infinity Cache cannot serve a launch
        sets = max(1, min(8, -(-1_500_000_000 // B2)))
        run2 = Runner(w2, dev, stream, sets=sets)
        steps2 = max(args.steps, 200)
        ms2, kms2 = run2.measure(steps2, max(args.warmup, 10))
        launch2 = percentiles_us(run2.distribution(steps2))
        sus2 = sustained(run2, kms2, B2)
        mix2 = None if args.no_copy_probe else mix_probe(w2, run2, stream)
        best2 = None if args.no_copy_probe else best_mix_probe(w2, run2, stream, mix2)
        dir2 = None if args.no_copy_probe else direction_probes(
            w2, [s_[0] for s_ in run2.sets], stream)
        del run2
        torch.cuda.empty_cache()
        secondary = {"workload": w2.name, "buffer_sets": sets, "steps": steps2,
                     "ms_per_step": round(ms2, 5), "kernel_ms": round(kms2, 5),
                     "launch_us": launch2, "sustained": sus2,
                     "achieved": round(B2 / (kms2 * 1e-3) / 1e9, 2), "unit": "GB/s",
                     "frac": round(B2 / (kms2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "tokens_per_s": round(w2.tokens / (kms2 * 1e-3), 1),
                     "plan": plan_of(w2),
                     "traffic": read_traffic(w2.name),
                     "row_mix_GBs": mix2,
                     "frac_of_row_mix_probe": None if mix2 is None else
                                              round(B2 / (kms2 * 1e-3) / 1e9 / mix2, 4),
                     "best_mix": best2,
                     "frac_of_best_mix": None if best2 is None else
                                         round(B2 / (kms2 * 1e-3) / 1e9 / best2["GBs"], 4),
                     "direction_probes": dir2,
                     "frac_of_serial": None if dir2 is None else
                                       round(B2 / (kms2 * 1e-3) / 1e9 / dir2["serial_GBs"], 4)}

    cpu = None
    parity = None
    if args.cpu_seconds > 0:   # before the variants, which overwrite the outputs
        cpu, parity = cpu_baseline(args, w, p, r, g, rout, nout, q, sc_out, sc_in)

    variants = None
    if not args.no_variants:
        variants = measure_variants(w, run, stream, max(args.steps, 10), args.warmup)

    decode = None
    if not args.no_variants:
        decode = decode_cold(stream)

    probes = None
    if not args.no_copy_probe:
        probes = hbm_probes(w, p, stream)

    plan = plan_of(w)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": w.partial_dtype if w.partial_dtype == w.act_dtype else
                    "%s partials, %s activations" % (w.partial_dtype, w.act_dtype),
        "data": "synthetic",
        "config": {"workload": w.name, "n_shards": w.n_shards, "tokens": t, "hidden": h,
                   "partial_dtype": w.partial_dtype, "act_dtype": w.act_dtype,
                   "quant": w.quant, "algorithmic_bytes": B},
        "tokens_per_s": round(t / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernel_ms": round(kernel_ms, 5),
        "launch_us": launch_us,
        "plan": plan,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "sustained": sus,
        "hbm_probes": probes,
        "frac_of_serial": None if probes is None else round(achieved / probes["serial_GBs"], 4),
        "frac_of_best_mix": None if probes is None else round(achieved / probes["best_mix_GBs"], 4),
        "frac_of_row_mix_probe": None if probes is None else round(achieved / probes["row_mix_GBs"], 4),
        "secondary": secondary,
        "variants": variants,
        "decode_cold": decode,
        "cpu_baseline": cpu,
        "sample_parity": parity,
    }
    print(json.dumps(line), flush=True)
    return 0


def sustained(run, kernel_ms, nbytes, seconds=1.0):
    """The same launches back to back for about ``seconds`` right after the timed region:
    the kernel's average duration once the GPU has been busy for a while. The timed steps
    follow a few seconds of start-up in which the GPU is mostly idle, and an MI355X that
    has just been idle runs these launches slightly faster (c4: about 482 against 484 us)."""
    n = max(20, min(20000, int(seconds / (kernel_ms * 1e-3))))
    _, ms = run.measure(n, 0)
    return {"launches": n, "kernel_ms": round(ms, 5),
            "achieved": round(nbytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def mix_probe(w, run, stream, reps=20):
    """The workload's own read/write mix with no arithmetic (GB/s), rotating over the
    runner's buffer sets like the timed launches: read a set's partials and write a
    buffer of its own in the workload's write:read ratio, one unit per row (reads, then
    writes, per unit)."""
    import torch

    import shard_reduce_residual_amd as arf

    n, t, h = w.n_shards, w.tokens, w.hidden
    B = w.algorithmic_bytes()
    alg_read = n * t * h * w.sp + t * h * w.sa + h * w.sa + (4 if w.quant == "per_tensor" else 0)
    read_b = n * t * h * w.sp
    write_b = (int(read_b * (B - alg_read) / alg_read) // 16) * 16
    outs = [torch.empty(write_b, dtype=torch.uint8, device=run.sets[0][0].device)
            for _ in run.sets]
    k = [0]

    def one():
        i = k[0] % len(run.sets)
        k[0] += 1
        arf.arf_stream_mix(outs[i], write_b, run.sets[i][0], read_b, units=t, stream=stream)

    ms = _events_ms(one, stream, reps, 3)
    del outs
    return round((read_b + write_b) / (ms * 1e-3) / 1e9, 1)


def best_mix_probe(w, run, stream, row_mix, reps=10):
    """The workload's read/write mix with no arithmetic as its best pattern (GB/s): the
    fastest of 1/32 .. 1/2 units per row (each unit reading its share before writing any)
    and the one-unit-per-row probe (row_mix, measured already), rotating over the runner's
    buffer sets like the timed launches."""
    import torch

    import shard_reduce_residual_amd as arf

    n, t, h = w.n_shards, w.tokens, w.hidden
    B = w.algorithmic_bytes()
    alg_read = n * t * h * w.sp + t * h * w.sa + h * w.sa + (4 if w.quant == "per_tensor" else 0)
    read_b = n * t * h * w.sp
    write_b = (int(read_b * (B - alg_read) / alg_read) // 16) * 16
    outs = [torch.empty(write_b, dtype=torch.uint8, device=run.sets[0][0].device)
            for _ in run.sets]
    best = {"GBs": row_mix, "units": t}
    for units in sorted({max(1, t // d) for d in (32, 16, 8, 4, 2)}):
        k = [0]

        def one():
            i = k[0] % len(run.sets)
            k[0] += 1
            arf.arf_stream_mix(outs[i], write_b, run.sets[i][0], read_b, units=units,
                               stream=stream)

        ms = _events_ms(one, stream, reps, 3)
        gbs = round((read_b + write_b) / (ms * 1e-3) / 1e9, 1)
        if gbs > best["GBs"]:
            best = {"GBs": gbs, "units": units}
    del outs
    return best


def _alg_split(w):
    """The workload's algorithmic bytes read and written per launch."""
    n, t, h = w.n_shards, w.tokens, w.hidden
    B = w.algorithmic_bytes()
    alg_read = n * t * h * w.sp + t * h * w.sa + h * w.sa + (4 if w.quant == "per_tensor" else 0)
    return alg_read, B - alg_read


UNIT_COUNTS = (256, 512, 1024, 2048, 4096)


def direction_probes(w, srcs, stream, reps=10):
    """Best read-only and write-only rates (GB/s) with no arithmetic, over several unit
    counts (256..4096 workgroups, and one per 16 KiB): reading each source buffer (the
    partials) in turn, and writing the workload's algorithmic write bytes to one buffer per
    source in turn, so that rotating sets larger than the 256 MB Infinity Cache are not
    served from it. serial_us is the time to read the workload's algorithmic read bytes at
    the read rate and then write its write bytes at the write rate: the pass with no
    overlap of reads and writes on the bus."""
    import torch

    import shard_reduce_residual_amd as arf

    alg_read, alg_write = _alg_split(w)
    read_b = srcs[0].numel() * srcs[0].element_size()
    write_b = (alg_write // 16) * 16
    dsts = [torch.empty(write_b, dtype=torch.uint8, device=srcs[0].device) for _ in srcs]

    def best(call):
        top = (0.0, 0)
        for units in UNIT_COUNTS + (0,):
            k = [0]

            def one():
                i = k[0] % len(srcs)
                k[0] += 1
                call(i, units)

            ms = _events_ms(one, stream, reps, 3)
            top = max(top, (1.0 / ms, units))
        return 1.0 / top[0], top[1]

    ms_r, u_r = best(lambda i, u: arf.arf_stream_mix(None, 0, srcs[i], read_b, units=u,
                                                     stream=stream))
    ms_w, u_w = best(lambda i, u: arf.arf_stream_mix(dsts[i], write_b, None, 0, units=u,
                                                     stream=stream))
    del dsts
    read_gbs = read_b / (ms_r * 1e-3) / 1e9
    write_gbs = write_b / (ms_w * 1e-3) / 1e9
    serial_us = (alg_read / read_gbs + alg_write / write_gbs) / 1e3
    return {"read_GBs": round(read_gbs, 1), "read_units": u_r or "per 16 KiB",
            "write_GBs": round(write_gbs, 1), "write_units": u_w or "per 16 KiB",
            "write_bytes": write_b, "serial_us": round(serial_us, 2),
            "serial_GBs": round(w.algorithmic_bytes() / (serial_us * 1e-6) / 1e9, 1)}


def hbm_probes(w, partials, stream, reps=10):
    """Streaming kernels with no arithmetic (GB/s): the best read-only and write-only rates
    and the serial pass they imply (direction_probes), a 1 GiB copy, and the workload's
    own read/write mix -- reading the partials buffer and writing a buffer in the
    workload's write:read ratio -- once as one unit per row (reads, then writes, per unit:
    row_mix) and once as the best over 1/32 .. 1 units per row (best_mix)."""
    import torch

    import shard_reduce_residual_amd as arf

    dev = partials.device
    read_b = partials.numel() * partials.element_size()
    t = w.tokens
    alg_read, alg_write = _alg_split(w)
    mix_write = (int(read_b * alg_write / alg_read) // 16) * 16
    out = direction_probes(w, [partials], stream, reps)
    one_gib = 1 << 30
    dst = torch.empty(max(mix_write, one_gib), dtype=torch.uint8, device=dev)
    flat = partials.view(torch.uint8).view(-1)
    # the copy probe moves 1 GiB: from the partials when they are that large, else from a
    # buffer of its own (its contents do not matter)
    src2 = (flat[:one_gib] if flat.numel() >= one_gib
            else torch.empty(one_gib, dtype=torch.uint8, device=dev))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_c = timed(lambda: arf.arf_stream_copy(dst, src2, one_gib, stream=stream))
    out["copy_GBs"] = round(2 * one_gib / t_c / 1e9, 1)
    t_m = timed(lambda: arf.arf_stream_mix(dst, mix_write, partials, read_b, units=t,
                                           stream=stream))
    out["row_mix_GBs"] = round((read_b + mix_write) / t_m / 1e9, 1)
    out["mix_read_fraction"] = round(read_b / (read_b + mix_write), 4)
    out["row_mix_units"] = t
    # the best pattern measured for this byte mix: fewer, larger units that each read all
    # of their share before writing any (with every unit resident, the whole chip reads and
    # then writes)
    best = (out["row_mix_GBs"], t)   # one unit per row is one of the patterns
    for units in sorted({max(1, t // d) for d in (32, 16, 8, 4, 2)}):
        tu = timed(lambda: arf.arf_stream_mix(dst, mix_write, partials, read_b, units=units,
                                              stream=stream))
        gbs = round((read_b + mix_write) / tu / 1e9, 1)
        if gbs > best[0]:
            best = (gbs, units)
    out["best_mix_GBs"], out["best_mix_units"] = best
    del dst
    return out


def _events_ms(fn, stream, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def graph_replay_us(launches=50, replays=20, repeats=7):
    """Per-launch time of the decode-size workloads (c0, c1, c2) when `launches` calls are
    captured in one HIP graph and the graph is replayed: the kernels' back-to-back time
    without host launch overhead. The replays are timed ``repeats`` times; the median is
    reported with the range, since single timings of µs-long kernels spread by about 10%."""
    import torch

    import workloads

    res = {}
    dev = torch.device("cuda:0")
    side = torch.cuda.Stream(device=dev)
    for key in ("c0", "c1", "c2"):
        w = workloads.WORKLOADS[key]
        run = Runner(w, dev, side, sets=1)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run.step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        run.stream = None   # launch on the capturing (current) stream
        with torch.cuda.graph(graph, stream=side):
            for _ in range(launches):
                run.step()
        graph.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / (replays * launches))
        times.sort()
        us = times[len(times) // 2]
        res[w.name] = {"us_per_launch": round(us, 3), "min": round(times[0], 3),
                       "max": round(times[-1], 3),
                       "achieved_GBs": round(w.algorithmic_bytes() / (us * 1e-6) / 1e9, 1)}
        del graph, run
    return res


def decode_cold(stream, launches=1000):
    """Per-launch time of the decode-size workloads (c0, c1, c2) with their inputs out of
    every cache: before each launch, outside its event pair, 1 GiB is written (four times
    the 256 MB Infinity Cache), then one 16-byte write lets that flush's end-of-kernel
    cache write-back finish before the first event. ``floor`` is a 16-byte write timed in
    the same position: the part of each figure that any launch there costs."""
    import torch

    import shard_reduce_residual_amd as arf
    import workloads

    dev = torch.device("cuda:0")
    one_gib = 1 << 30
    junk = torch.empty(one_gib, dtype=torch.uint8, device=dev)

    def flush():
        arf.arf_stream_mix(junk, one_gib, None, 0, stream=stream)
        arf.arf_stream_mix(junk, 16, None, 0, stream=stream)

    class Tiny:   # a one-workgroup, 16-byte write: what any launch costs in this position
        def __init__(self):
            self.stream = stream

        def step(self):
            arf.arf_stream_mix(junk, 16, None, 0, stream=stream)

    res = {"floor": percentiles_us(Runner.distribution(Tiny(), launches, flush=flush))}
    for key in ("c0", "c1", "c2"):
        w = workloads.WORKLOADS[key]
        run = Runner(w, dev, stream, sets=1)
        for _ in range(5):
            run.step()
        us = percentiles_us(run.distribution(launches, flush=flush))
        us["achieved_GBs_at_median"] = round(w.algorithmic_bytes() / (us["median"] * 1e-6) / 1e9, 1)
        res[w.name] = us
        del run
    del junk
    torch.cuda.empty_cache()
    return res


def measure_variants(w, run, stream, steps, warmup):
    """The same workload with accumulation in the partial type, and one rank's share of
    the token-slice exchange (reduce T/N rows of the N shards; then the epilogue over
    all T rows from the gathered reduced values, as one shard)."""
    import torch

    import shard_reduce_residual_amd as arf

    p, r, g, rout, nout, q, sc_out, sc_in = run.sets[0]
    t, h, n = w.tokens, w.hidden, w.n_shards
    mode = arf.ARF_QUANT_PER_TOKEN if w.quant == "per_token" else arf.ARF_QUANT_PER_TENSOR
    quant = dict(quant_out=q, mode=mode, scale_in=sc_in, scale_out=sc_out) if w.quant else {}
    B = w.algorithmic_bytes()
    out = {}

    def acc_partial():
        arf.arf_fused_epilogue(p, r, g, w.eps, residual_out=rout, norm_out=nout,
                               accumulate=arf.ARF_ACC_PARTIAL, stream=stream, **quant)

    ms = _events_ms(acc_partial, stream, steps, warmup)
    out["accumulate_partial"] = {"kernel_ms": round(ms, 5),
                                 "achieved": round(B / (ms * 1e-3) / 1e9, 2)}

    sums = torch.empty((t, h), dtype=rout.dtype, device=rout.device)
    cnt = t // n + (1 if t % n else 0)   # rank 0's slice (the largest)

    def reduce_slice():
        arf.arf_reduce_rows(p, sums, row_begin=0, row_count=cnt, stream=stream)

    def epilogue():
        arf.arf_reduce_add_rmsnorm_quant(sums.view(1, t, h), r, g, w.eps, q, mode,
                                         scale_in=sc_in, scale_out=sc_out, residual_out=rout,
                                         norm_out=nout, stream=stream) if w.quant else \
            arf.arf_reduce_add_rmsnorm(sums.view(1, t, h), r, g, w.eps, residual_out=rout,
                                       norm_out=nout, stream=stream)

    arf.arf_reduce_rows(p, sums, stream=stream)   # every row holds a reduced value
    ms_r = _events_ms(reduce_slice, stream, steps, warmup)
    ms_e = _events_ms(epilogue, stream, steps, warmup)
    sp = w.sp
    b_r = n * cnt * h * sp + cnt * h * 2
    b_e = w.with_tokens(t).algorithmic_bytes() - n * t * h * sp + t * h * 2
    out["token_slice_share"] = {
        "slice_rows": cnt, "reduce_ms": round(ms_r, 5),
        "reduce_achieved": round(b_r / (ms_r * 1e-3) / 1e9, 2),
        "epilogue_ms": round(ms_e, 5), "epilogue_achieved": round(b_e / (ms_e * 1e-3) / 1e9, 2),
        "unit": "GB/s"}
    del sums

    # decode-size calls replayed from a HIP graph (no per-launch host overhead)
    out["graph_replay"] = graph_replay_us()

    # the block-scaled 4-bit copy in place of the fp8 one
    if h % 32 == 0:
        q4 = torch.empty((t, h // 2), dtype=torch.uint8, device=rout.device)
        s4 = torch.empty((t, h // 32), dtype=torch.uint8, device=rout.device)

        def mx():
            arf.arf_fused_epilogue(p, r, g, w.eps, residual_out=rout, norm_out=nout,
                                   quant_out=q4, mode=arf.ARF_QUANT_MXFP4, scale_out=s4,
                                   stream=stream)

        ms = _events_ms(mx, stream, steps, warmup)
        b_mx = (w.with_tokens(t).algorithmic_bytes() - (t * h + 4 * t if w.quant == "per_token"
                                                         else (t * h + 4 if w.quant else 0))
                + t * h // 2 + t * h // 32)
        out["mxfp4"] = {"kernel_ms": round(ms, 5), "algorithmic_bytes": b_mx,
                        "achieved": round(b_mx / (ms * 1e-3) / 1e9, 2), "unit": "GB/s"}
        del q4, s4
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(args, w, p, r, g, rout, nout, q, sc_out, sc_in):
    """Oracle on the first rows of the same workload, on the host's cores, repeated until
    about --cpu-seconds of work; also checks the GPU's outputs for those rows."""
    import numpy as np

    import oracle
    import workloads

    rows = min(w.tokens, 1024)
    ph = workloads.to_bits(p[:, :rows].contiguous())
    rh = workloads.to_bits(r[:rows].contiguous())
    gh = workloads.to_bits(g)
    threads = min(16, oracle.default_threads())
    kw = dict(partial_dtype=w.partial_dtype, act_dtype=w.act_dtype, quant=w.quant,
              n_threads=threads)
    if w.quant == "per_tensor":
        kw["scale_in"] = float(sc_in.item())
    oracle.lib()
    passes, elapsed, ref = 0, 0.0, None
    while elapsed < args.cpu_seconds and passes < 200:
        s = time.perf_counter()
        ref = oracle.reduce_add_rmsnorm(ph, rh, gh, w.eps, **kw)
        elapsed += time.perf_counter() - s
        passes += 1
    sample_bytes = w.with_tokens(rows).algorithmic_bytes()
    # the same oracle on one thread, over the first eighth of those rows
    rows1 = max(1, rows // 8)
    kw1 = dict(kw, n_threads=1)
    p1, r1 = ph[:, :rows1].copy(), rh[:rows1].copy()
    passes1, elapsed1 = 0, 0.0
    while elapsed1 < args.cpu_seconds / 4 and passes1 < 200:
        s = time.perf_counter()
        oracle.reduce_add_rmsnorm(p1, r1, gh, w.eps, **kw1)
        elapsed1 += time.perf_counter() - s
        passes1 += 1
    cpu = {"value": round(sample_bytes * passes / elapsed / 1e9, 3), "unit": "GB/s",
           "tokens_per_s": round(rows * passes / elapsed, 1), "cores": threads,
           "kind": "oracle",
           "sample": "first %d of %d tokens of %s, %d passes, %.1f s"
                     % (rows, w.tokens, w.name, passes, elapsed),
           "one_thread": {"value": round(w.with_tokens(rows1).algorithmic_bytes() * passes1
                                         / elapsed1 / 1e9, 3),
                          "tokens_per_s": round(rows1 * passes1 / elapsed1, 1),
                          "sample": "first %d tokens, %d passes, %.1f s"
                                    % (rows1, passes1, elapsed1)},
           "cpu_model": cpu_model(), "host_cpus": oracle.default_threads()}

    def ordinal(b, bits):
        b = b.astype(np.int64)
        s = 1 << (bits - 1)
        return np.where(b & s, -(b & (s - 1)), b)

    gr = workloads.to_bits(rout[:rows])
    gn = workloads.to_bits(nout[:rows])
    par = {"rows": rows,
           "residual_bit_exact": bool(np.array_equal(gr, ref["residual_out"])),
           "norm_max_ulp": int(np.abs(ordinal(gn, 16) - ordinal(ref["norm_out"], 16)).max())}
    if q is not None:
        gq = q[:rows].cpu().numpy()
        par["fp8_max_code_diff"] = int(np.abs(ordinal(gq, 8) - ordinal(ref["quant_out"], 8)).max())
    return cpu, par


if __name__ == "__main__":
    sys.exit(main())
