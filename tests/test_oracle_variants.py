"""Pins for the oracle's variants (CPU only): accumulation in the partial type, row
ranges, and the reduce-only share of the token-slice exchange.

Method: TensorRT-LLM page "allReduceFusionKernels.cu": allreduce_sum (both branches);
the twoshot kernel (a rank reduces its slice of tokens, then every rank runs the fused
epilogue over the reduced values) and the launcher's slice arithmetic.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import act_bits_to_f64, exact_to_act_bits, ordinal16, read_golden


def _bits(values, act):
    return exact_to_act_bits(np.asarray(values, dtype=np.float64), act)


def test_partial_accumulation_golden():
    rows = read_golden("partial_accumulation.txt")
    assert len(rows) == 5
    for act, acc, *vals in rows:
        p = [float(v) for v in vals[:4]]
        want = float(vals[4])
        h = 8
        part = np.stack([np.full((1, h), _bits([v], act)[0], np.uint16) for v in p])
        zero = np.zeros((1, h), np.uint16)
        gam = np.full((h,), _bits([1.0], act)[0], np.uint16)
        out = oracle.reduce_add_rmsnorm(part, zero, gam, 1e-6, partial_dtype=act, act_dtype=act,
                                        accumulate=acc)
        got = act_bits_to_f64(out["residual_out"], act)
        assert np.all(got == want), (act, acc, p, got[0, 0])
        sums = oracle.reduce_rows(part, partial_dtype=act, act_dtype=act, accumulate=acc)
        assert np.all(act_bits_to_f64(sums, act) == want)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_partial_accumulation_step_by_step(act, n):
    # Partials k * 2^-4: every pairwise sum is exact in fp32, so each step's rounding is a
    # library cast of the exact sum.
    rng = np.random.default_rng(40 + n)
    kmax = 127 if act == "bf16" else 1023
    t, h = 3, 64
    pv = rng.integers(-kmax, kmax + 1, size=(n, t, h)).astype(np.float64) * 2.0 ** -4
    pb = _bits(pv, act)
    acc = act_bits_to_f64(pb[0], act)
    for r in range(1, n):
        acc = act_bits_to_f64(exact_to_act_bits(acc + act_bits_to_f64(pb[r], act), act), act)
    sums = oracle.reduce_rows(pb, partial_dtype=act, act_dtype=act, accumulate="partial")
    assert np.array_equal(act_bits_to_f64(sums, act), acc)
    # and the fp32 branch rounds only once
    sums32 = oracle.reduce_rows(pb, partial_dtype=act, act_dtype=act, accumulate="f32")
    assert np.array_equal(sums32, exact_to_act_bits(pv.sum(axis=0), act))
    if n >= 8:   # partial sums outgrow the 16-bit mantissa, so the branches differ
        assert not np.array_equal(sums, sums32)


def test_partial_accumulation_is_fp32_for_fp32_partials():
    w = workloads.WORKLOADS["c3"].with_tokens(3)
    p, r, g = (workloads.to_bits(x) for x in workloads.generate(w, "cpu"))
    a = oracle.reduce_add_rmsnorm(p, r, g, w.eps, partial_dtype="f32", act_dtype="bf16")
    b = oracle.reduce_add_rmsnorm(p, r, g, w.eps, partial_dtype="f32", act_dtype="bf16",
                                  accumulate="partial")
    for k in a:
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("begin,count", [(0, 5), (3, 4), (7, -1), (11, 0), (0, -1)])
def test_row_range_matches_full_run_and_leaves_other_rows(begin, count):
    w = workloads.WORKLOADS["c1"].with_tokens(11)
    p, r, g = (workloads.to_bits(x) for x in workloads.generate(w, "cpu"))
    full = oracle.reduce_add_rmsnorm(p, r, g, w.eps, partial_dtype="bf16", act_dtype="bf16",
                                     quant="per_token")
    part = oracle.reduce_add_rmsnorm(p, r, g, w.eps, partial_dtype="bf16", act_dtype="bf16",
                                     quant="per_token", rows=(begin, count), out_init=0xA5)
    end = 11 if count < 0 else begin + count
    for k in full:
        assert np.array_equal(part[k][begin:end], full[k][begin:end])
        outside = np.concatenate([part[k][:begin].ravel().view(np.uint8),
                                  part[k][end:].ravel().view(np.uint8)])
        assert np.all(outside == 0xA5)


def test_reduce_rows_is_the_residual_out_of_a_zero_residual():
    w = workloads.WORKLOADS["c2"].with_tokens(6)
    p, r, g = (workloads.to_bits(x) for x in workloads.generate(w, "cpu"))
    zero = np.zeros_like(r)
    full = oracle.reduce_add_rmsnorm(p, zero, g, w.eps, partial_dtype="bf16", act_dtype="bf16")
    sums = oracle.reduce_rows(p, partial_dtype="bf16", act_dtype="bf16")
    # s + (+0) = s except that -0 + +0 = +0
    assert np.array_equal(ordinal16(sums), ordinal16(full["residual_out"]))
    # the twoshot composition: reduce every slice, then the epilogue with N = 1 over the
    # reduced values gives the oneshot result bit for bit
    n = w.n_shards
    t = w.tokens
    gathered = np.full((t, w.hidden), 0xFFFF, np.uint16)
    for rank in range(n):   # the page's launcher: t // n rows each, the first t % n get one more
        cnt = t // n + (1 if rank < t % n else 0)
        beg = rank * (t // n) + min(rank, t % n)
        s = oracle.reduce_rows(p, partial_dtype="bf16", act_dtype="bf16", rows=(beg, cnt))
        gathered[beg:beg + cnt] = s[beg:beg + cnt]
    assert not np.any(gathered == 0xFFFF)
    two = oracle.reduce_add_rmsnorm(gathered[None], r, g, w.eps, partial_dtype="bf16",
                                    act_dtype="bf16", quant="per_token")
    one = oracle.reduce_add_rmsnorm(p, r, g, w.eps, partial_dtype="bf16", act_dtype="bf16",
                                    quant="per_token")
    for k in one:
        assert np.array_equal(two[k], one[k])


def test_variant_argument_errors():
    p = np.zeros((2, 4, 8), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.reduce_rows(p, partial_dtype="bf16", act_dtype="bf16", rows=(3, 2))
    with pytest.raises(oracle.OracleError):
        oracle.reduce_rows(p, partial_dtype="bf16", act_dtype="bf16", rows=(-1, 1))
    L = oracle.lib()
    assert L.arfo_reduce_rows(p.ctypes.data, 2, 4, 8, 0, 0, 7, 0, -1, p.ctypes.data, 1) == 4
