"""Pins for the oracle's scalar conversions (CPU only).

Each conversion is checked against something other than itself:
  * fp32 -> bf16 against torch's own cast, on every bf16 binade's ties and near-ties;
  * fp32 -> f16 against numpy's own cast, same construction;
  * fp32 -> E4M3 against a brute-force nearest-value search over the 127 finite
    magnitudes of the OFP8 definition, against torch's float8_e4m3fn cast inside the
    finite range, and against the hand-derived fixed points in golden/.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (e4m3_brute, e4m3_code_to_f64, e4m3_values, numpy_f16_bits,
                     read_golden, torch_bf16_bits)

RNG = np.random.default_rng(1234)


def _random_f32(n, rng=RNG):
    return rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def test_bf16_cast_matches_torch_on_every_tie():
    # For every bf16 pattern, probe the fp32 values whose low 16 bits are 0, 1, the tie
    # 0x8000 and its neighbours, and all-ones: every rounding decision in every binade.
    hi = np.arange(0x10000, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                    np.uint32)
    x = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    x = np.concatenate([x, _random_f32(1 << 20)])
    got = oracle.f32_to_bf16(x)
    want = torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    # NaN stays NaN (quiet): exponent all ones and a non-zero mantissa with the quiet bit
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all(got[nan] & 0x0040)


def test_f16_cast_matches_numpy_on_every_tie():
    # All binary16 patterns, their midpoints to the next pattern (exact in fp32), and
    # one fp32 ulp either side of each midpoint.
    h = np.arange(0x7C00, dtype=np.uint16)                    # +0 .. largest finite
    v = h.view(np.float16).astype(np.float32)
    nxt = (h + 1).view(np.float16).astype(np.float32)         # 0x7C00 is +inf
    mid = np.where(np.isinf(nxt), np.float32(65520.0), (v.astype(np.float64) + nxt) / 2).astype(np.float32)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    x = np.concatenate([v, mid, below, above])
    x = np.concatenate([x, -x, _random_f32(1 << 20),
                        np.array([np.inf, -np.inf, 1e30, -1e30, 65519.996, 65520.0], np.float32)])
    got = oracle.f32_to_f16(x)
    want = numpy_f16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all(got[nan] & 0x0200)


def _e4m3_probe_points():
    vals = e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2                         # exact in fp32
    pts = np.concatenate([vals, mids, [448 + 16, 448 + 8, 480, 1e4]]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(0)),
                          np.nextafter(pts, np.float32(np.inf))])
    logu = np.exp2(RNG.uniform(-14, 10, size=200_000)).astype(np.float32)
    pts = np.concatenate([pts, logu])
    return np.concatenate([pts, -pts])


def test_e4m3_cast_matches_brute_force_nearest():
    x = _e4m3_probe_points()
    x = np.concatenate([x, _random_f32(100_000),
                        np.array([np.inf, -np.inf, np.nan, 0.0, -0.0], np.float32)])
    got = oracle.f32_to_e4m3(x)
    want = e4m3_brute(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_e4m3_cast_matches_torch_in_finite_range():
    x = _e4m3_probe_points()
    x = x[np.abs(x) <= 448]
    got = oracle.f32_to_e4m3(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_golden_fixed_points():
    rows = read_golden("e4m3_fixed_points.txt")
    assert len(rows) >= 15
    x = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    assert np.array_equal(oracle.f32_to_e4m3(x), want)


def test_decoders_invert_encoders():
    codes = np.arange(256, dtype=np.uint8)
    dec = oracle.e4m3_to_f32(codes)
    ref = e4m3_code_to_f64(codes)
    fin = ~np.isnan(ref)
    assert np.array_equal(dec[fin].astype(np.float64), ref[fin])
    assert np.all(np.isnan(dec[~fin])) and set(codes[~fin]) == {0x7F, 0xFF}
    back = oracle.f32_to_e4m3(dec[fin])
    assert np.array_equal(back, codes[fin])
    h = np.arange(0x10000, dtype=np.uint16)
    f = oracle.f16_to_f32(h[::7])
    assert np.array_equal(f[~np.isnan(f)], h[::7].view(np.float16).astype(np.float32)[~np.isnan(f)])


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_scalar_entry_points_agree_with_bulk(act):
    x = _random_f32(4096)
    L = oracle.lib()
    f = L.arfo_f32_to_bf16 if act == "bf16" else L.arfo_f32_to_f16
    bulk = oracle.f32_to_bf16(x) if act == "bf16" else oracle.f32_to_f16(x)
    assert [f(float(v)) for v in x] == list(bulk)
