"""The seeded input generator (CPU): SplitMix64 elements against their definition in
Python integers and against the generator's published reference outputs, the Box-Muller
pairs against their uniforms, and the workload recipe's shapes and moments."""
import math
import os

import numpy as np
import torch

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def test_raw64_matches_the_integer_definition_with_wraparound():
    for seed in (0, 1, 4, 1234567, 2 ** 63 + 12345, 2 ** 64 - 1):
        for stream in (0, 1, 2, 3):
            for start in (0, 999, (1 << 40) - 8):
                got = workloads.raw64(seed, stream, start, 8, "cpu").tolist()
                want = [workloads.raw64_reference(seed, stream, start + i) for i in range(8)]
                assert [v & workloads._MASK64 for v in got] == want, (seed, stream, start)


def test_raw64_reproduces_the_reference_splitmix64_sequence():
    # tests/golden/splitmix64_seed1234567.txt: the first outputs of SplitMix64 seeded with
    # 1234567, as reproduced by public SplitMix64 implementations; element n of stream 0
    # is output n + 1 of that sequence
    vals = [int(l.split()[1]) for l in open(os.path.join(HERE, "golden", "splitmix64_seed1234567.txt"))
            if l.strip() and not l.startswith("#")]
    got = workloads.raw64(1234567, 0, 0, len(vals), "cpu").tolist()
    assert [v & workloads._MASK64 for v in got] == vals


def test_box_muller_pairs_follow_their_uniforms():
    u = workloads.uniform(7, 0, 0, 2000, "cpu").numpy().reshape(-1, 2)
    z = workloads.normal(7, 0, 0, 2000, "cpu").numpy().reshape(-1, 2)
    assert np.all((u >= 0) & (u < 1))
    r2 = -2.0 * np.log(1.0 - u[:, 0])
    assert np.allclose(z[:, 0] ** 2 + z[:, 1] ** 2, r2, rtol=1e-12, atol=1e-300)
    ang = np.arctan2(z[:, 1], z[:, 0]) % (2 * math.pi)
    assert np.allclose(ang, (2 * math.pi * u[:, 1]) % (2 * math.pi), atol=1e-9)
    # an offset window gives the same elements as the full draw
    assert np.array_equal(workloads.normal(7, 0, 600, 400, "cpu").numpy(), z.reshape(-1)[600:1000])


def test_workload_recipe_moments_and_outliers():
    w = workloads.WORKLOADS["c3"].with_tokens(64)
    p, r, g = workloads.generate(w, "cpu")
    assert p.dtype == torch.float32 and r.dtype == torch.bfloat16 and g.dtype == torch.bfloat16
    cols = workloads.outlier_channels(w)
    assert cols.numel() == 72 and len(set(cols.tolist())) == 72
    mask = torch.zeros(w.hidden, dtype=torch.bool)
    mask[cols] = True
    assert abs(p[:, :, ~mask].std().item() - 1.0) < 0.01
    assert abs(p[:, :, mask].std().item() - 100.0) < 2.0
    assert abs(r.float().std().item() - 1.0) < 0.01
    assert 0.5 <= g.float().min().item() and g.float().max().item() <= 1.5


def test_row_generator_matches_the_whole_generator():
    # generate_rows gives exactly the rows of generate, outlier channels included
    for key in ("c0", "c3"):
        w = workloads.WORKLOADS[key].with_tokens(40)
        p, r, g = workloads.generate(w, "cpu")
        for b, c in ((0, 7), (13, 20), (39, 1)):
            pr, rr, gr = workloads.generate_rows(w, b, c, "cpu")
            assert torch.equal(pr, p[:, b:b + c]) and torch.equal(rr, r[b:b + c])
            assert torch.equal(gr, g)
