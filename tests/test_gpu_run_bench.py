"""The benchmark end to end on a small workload (GPU): one JSON line with the fields the
benchmark contract names, a roofline object from the events, the oracle baseline, and
sample parity of the timed outputs against the oracle."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_contract_line():
    print("[case] bench.py --workload c1 --secondary c2", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "c1",
                        "--secondary", "c2", "--steps", "5", "--warmup", "2",
                        "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["value"] > 0
    assert d["config"]["workload"] == "c1_n8_t128_h4096_bf16"
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    sp = d["sample_parity"]
    assert sp["residual_bit_exact"] and sp["norm_max_ulp"] <= 1
    # the probes: the kernel's own row-by-row mix, and the best pattern for the same byte
    # mix, which the row-by-row probe cannot beat
    hp = d["hbm_probes"]
    assert hp["best_mix_GBs"] >= hp["row_mix_GBs"] > 0 and hp["best_mix_units"] >= 1
    assert abs(d["frac_of_best_mix"] - rl["achieved"] / hp["best_mix_GBs"]) < 1e-3
    # the best single-direction rates and the serial pass they imply
    assert hp["read_GBs"] > 0 and hp["write_GBs"] > 0 and hp["serial_us"] > 0
    serial_gbs = d["config"]["algorithmic_bytes"] / (hp["serial_us"] * 1e-6) / 1e9
    assert abs(serial_gbs / hp["serial_GBs"] - 1) < 1e-3
    assert abs(d["frac_of_serial"] - rl["achieved"] / hp["serial_GBs"]) < 1e-3
    assert d["secondary"]["direction_probes"]["serial_GBs"] > 0
    # the same launches back to back for about a second after the timed region
    for sus in (d["sustained"], d["secondary"]["sustained"]):
        assert sus["launches"] >= 20 and sus["kernel_ms"] > 0
        assert abs(sus["frac"] - sus["achieved"] / rl["peak"]) < 1e-3
    assert d["secondary"]["workload"] == "c2_n8_t64_h8192_bf16_fp8tensor"
    assert d["secondary"]["best_mix"]["GBs"] > 0
    for key in ("c0_n2_t16_h1024_bf16", "c1_n8_t128_h4096_bf16",
                "c2_n8_t64_h8192_bf16_fp8tensor"):
        assert d["variants"]["graph_replay"][key]["us_per_launch"] > 0
        assert d["decode_cold"][key]["median"] > 0


def test_bench_refuses_more_than_one_gpu():
    # CPU: the refusal comes before anything touches a device
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout.strip()
