"""Test-side helpers: comparisons and independent reference roundings.

Nothing here implements the method; these are the yardsticks the oracle and the HIP
path are measured with (ordinal ulp distance, library casts, brute-force E4M3).
"""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def ordinal16(bits):
    """Monotone integer map of 16-bit float patterns; +0 and -0 both map to 0."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ordinal8(codes):
    q = np.asarray(codes, dtype=np.uint8).astype(np.int32)
    return np.where(q & 0x80, -(q & 0x7F), q)


def ulp_diff16(a, b):
    return np.abs(ordinal16(a) - ordinal16(b))


def code_diff8(a, b):
    return np.abs(ordinal8(a) - ordinal8(b))


# ---- library casts used as independent references ------------------------------------

def torch_bf16_bits(x_f32):
    """fp32 -> bf16 by torch's own cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def numpy_f16_bits(x):
    """fp32 or fp64 -> binary16 by numpy's cast (round to nearest even, one rounding;
    overflow to +-inf is intended, so numpy's overflow warning is silenced)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x).astype(np.float16).view(np.uint16)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def act_bits_to_f64(b, act):
    return bf16_bits_to_f64(b) if act == "bf16" else f16_bits_to_f64(b)


def act_ulp(v, act):
    """Spacing of the activation type at the magnitude of v (v in its normal range)."""
    mb, emin = (7, -126) if act == "bf16" else (10, -14)
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return np.exp2(e - mb)


def exact_to_act_bits(v64, act):
    """Correctly rounded cast of fp64 values that are exact in fp32 (asserted) to the
    activation type: torch's fp32->bf16 cast, or numpy's direct fp64->f16 cast."""
    v64 = np.asarray(v64, dtype=np.float64)
    if act == "bf16":
        v32 = v64.astype(np.float32)
        assert np.array_equal(v32.astype(np.float64), v64), "value not exact in fp32"
        return torch_bf16_bits(v32)
    return numpy_f16_bits(v64)


# ---- E4M3 by brute force over its finite values ----------------------------------------

def e4m3_values():
    """Values of codes 0x00..0x7E from the OFP8 E4M3 definition (bias 7, 3 mantissa
    bits; exponent field 0 is subnormal: m * 2^-9)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, np.float64)


_E4M3 = e4m3_values()


def e4m3_brute(x):
    """Nearest finite E4M3 value, ties to the even code, saturating at 448; +-inf -> +-448;
    NaN -> S.1111.111. Sign is kept (tiny negatives give -0 = 0x80)."""
    with np.errstate(over="ignore", invalid="ignore"):   # inf and NaN inputs are intended
        x = np.asarray(x, dtype=np.float32).astype(np.float64).ravel()
    out = np.empty(x.size, np.uint8)
    for s in range(0, x.size, 65536):
        xs = x[s:s + 65536]
        a = np.abs(xs)
        # beyond 2048 every finite candidate but 448 is farther away; clamping keeps the
        # fp64 distances distinguishable for huge inputs and infinities
        a = np.minimum(a, 2048.0)
        d = np.abs(a[:, None] - _E4M3[None, :])
        d = np.where(np.isnan(d), np.inf, d)
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among the (at most two) nearest codes prefer the even one
        even = cand & ((np.arange(0x7F) & 1) == 0)[None, :]
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        code = pick.astype(np.uint8)
        code = np.where(np.signbit(xs), code | 0x80, code).astype(np.uint8)
        code = np.where(np.isnan(xs), np.where(np.signbit(xs), 0xFF, 0x7F), code)
        out[s:s + 65536] = code
    return out


def e4m3_code_to_f64(q):
    q = np.asarray(q, dtype=np.uint8)
    mag = _E4M3[np.minimum(q & 0x7F, 0x7E)]
    mag = np.where((q & 0x7F) == 0x7F, np.nan, mag)
    return np.where(q & 0x80, -mag, mag)


# ---- OCP MX FP4 (E2M1) by brute force ------------------------------------------------------

_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # codes 0..7 (MX v1.0 table)


def e2m1_brute(x):
    """Nearest E2M1 magnitude, ties to the even code, saturating at 6; sign in bit 3."""
    x = np.asarray(x, dtype=np.float64).ravel()
    a = np.minimum(np.abs(x), 64.0)
    d = np.abs(a[:, None] - _E2M1[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & ((np.arange(8) & 1) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)
    return np.where(np.signbit(x), pick | 0x8, pick).astype(np.uint8)


def e2m1_code_to_f64(q):
    q = np.asarray(q, dtype=np.uint8)
    mag = _E2M1[q & 0x7]
    return np.where(q & 0x8, -mag, mag)


def unpack_fp4(packed):
    """[..., H/2] bytes -> [..., H] codes (element 2k in the low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
