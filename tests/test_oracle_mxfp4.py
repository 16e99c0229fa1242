"""Pins for the oracle's MXFP4 copy (CPU only).

OCP Microscaling Formats (MX) v1.0: MXFP4 blocks of 32 E2M1 elements share an E8M0 scale
X = 2^(floor(log2(max|V|)) - 2); elements are V / X rounded to nearest even, saturating at 6.
Checked against a brute-force nearest search over the 8 E2M1 magnitudes, hand-derived fixed
points (golden/mxfp4_fixed_points.txt), the scale definition, and dequantisation bounds.
"""
import numpy as np

import oracle
import workloads
from helpers import (act_bits_to_f64, e2m1_brute, e2m1_code_to_f64, read_golden,
                     unpack_fp4)


def test_e2m1_golden_fixed_points():
    rows = read_golden("mxfp4_fixed_points.txt")
    x = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    assert np.array_equal(oracle.f32_to_e2m1(x), want)


def test_e2m1_matches_brute_force():
    rng = np.random.default_rng(7)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    pts = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10),
                          [0, 0.5, 1, 1.5, 2, 3, 4, 6, 6.5, 7, 100],
                          rng.uniform(0, 8, 20000), np.exp2(rng.uniform(-12, 4, 5000))])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    assert np.array_equal(oracle.f32_to_e2m1(pts), e2m1_brute(pts))
    codes = np.arange(16, dtype=np.uint8)
    dec = np.array([oracle.lib().arfo_e2m1_to_f32(int(c)) for c in codes])
    assert np.array_equal(dec, e2m1_code_to_f64(codes))


def test_scale_code_definition():
    # E8M0 code = 127 + floor(log2 amax) - 2, clamped; amax == 0 -> 0
    cases = {1.0: 125, 6.0: 127, 7.99: 127, 8.0: 128, 0.5: 124, 2.0 ** -120: 5,
             2.0 ** -130: 0, 0.0: 0, 3.0e38: 252}
    for amax, code in cases.items():
        assert oracle.mx_scale_code(np.float32(amax)) == code, amax


def _run(key, tokens):
    w = workloads.WORKLOADS[key].with_tokens(tokens)
    p, r, g = (workloads.to_bits(x) for x in workloads.generate(w, "cpu"))
    return w, oracle.reduce_add_rmsnorm(p, r, g, w.eps, partial_dtype=w.partial_dtype,
                                        act_dtype=w.act_dtype, quant="mxfp4")


def test_mxfp4_blocks_follow_the_definition():
    w, out = _run("c1", 5)
    y = act_bits_to_f64(out["norm_out"], "bf16")
    t, h = y.shape
    codes = unpack_fp4(out["quant_out"])
    assert codes.shape == (t, h) and out["scale_out"].shape == (t, h // 32)
    blocks = y.reshape(t, h // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    shared = np.floor(np.log2(amax)) - 2
    assert np.array_equal(out["scale_out"].astype(np.int64), (shared + 127).astype(np.int64))
    X = np.exp2(shared)[:, :, None]
    want = e2m1_brute((blocks / X).ravel()).reshape(t, h)
    assert np.array_equal(codes, want)
    # the block maximum lands on 4 or 6 (amax / X is in [4, 8))
    top = np.abs(blocks) == amax[:, :, None]
    assert np.all(np.isin(codes.reshape(t, h // 32, 32)[top] & 0x7, [6, 7]))
    # dequantisation error: a quarter of |y| for normal codes, X/4 below 1, 2X above 6
    deq = e2m1_code_to_f64(codes).reshape(t, h // 32, 32) * X
    v = np.abs(blocks / X)
    err = np.abs(deq - blocks) / X
    assert np.all(err[(v >= 1) & (v <= 6)] <= v[(v >= 1) & (v <= 6)] / 4 + 1e-12)
    assert np.all(err[v < 1] <= 0.25 + 1e-12)
    assert np.all(err[v > 6] <= 2.0 + 1e-12)


def test_mxfp4_zero_block_and_shape_error():
    h = 64
    zero = np.zeros((1, 2, h), np.uint16)
    g = np.full((h,), 0x3F80, np.uint16)
    out = oracle.reduce_add_rmsnorm(zero, zero[0], g, 1e-6, partial_dtype="bf16",
                                    act_dtype="bf16", quant="mxfp4")
    assert np.all(out["scale_out"] == 0) and np.all(out["quant_out"] == 0)
    import pytest
    with pytest.raises(oracle.OracleError):
        oracle.reduce_add_rmsnorm(np.zeros((1, 2, 48), np.uint16), np.zeros((2, 48), np.uint16),
                                  np.zeros(48, np.uint16), 1e-6, partial_dtype="bf16",
                                  act_dtype="bf16", quant="mxfp4")
