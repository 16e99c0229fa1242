"""Pins for the oracle's fused epilogue (CPU only).

Each test fixes part of the pipeline with something other than the oracle itself:
hand-derived vectors (golden/), exact arithmetic on tiny inputs cast by torch/numpy,
the textbook RMSNorm in fp64, and invariants that hold for the exact method
(N=1 identity, gamma=1 unit RMS, power-of-two scaling, channel permutation, thread
count, the fp8 amax code and dequantisation bound).

Method: TensorRT-LLM page "allReduceFusionKernels.cu" (allreduce_sum fp32 branch,
fused_op/add128, rms_norm); FlashInfer page for
trtllm_create_ipc_workspace_for_all_reduce_fusion ([N][T][H] shards, fp32 option).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (act_bits_to_f64, act_ulp, code_diff8, e4m3_brute, e4m3_code_to_f64,
                     exact_to_act_bits, numpy_f16_bits, ordinal16, read_golden,
                     torch_bf16_bits, ulp_diff16)


def _act_bits(values, act):
    v = np.asarray(values, dtype=np.float64)
    return exact_to_act_bits(v, act)


def _run(p, res, gamma, eps, pd, ad, **kw):
    return oracle.reduce_add_rmsnorm(p, res, gamma, eps, partial_dtype=pd, act_dtype=ad, **kw)


# ---- hand-derived vectors --------------------------------------------------------------

def test_rank_order_golden():
    for row in read_golden("order_sensitivity.txt"):
        p = [float(v) for v in row[:4]]
        res, want = float(row[4]), float(row[5])
        h = 8
        part = np.stack([np.full((1, h), _act_bits([v], "bf16")[0], np.uint16) for v in p])
        resb = np.full((1, h), _act_bits([res], "bf16")[0], np.uint16)
        gam = np.full((h,), _act_bits([1.0], "bf16")[0], np.uint16)
        out = _run(part, resb, gam, 1e-6, "bf16", "bf16")
        got = act_bits_to_f64(out["residual_out"], "bf16")
        assert np.all(got == want), (row, got[0, 0])


def test_rne_ties_golden():
    for act, p0, res, want in read_golden("rne_ties.txt"):
        h = 16
        part = np.full((1, 1, h), _act_bits([float(p0)], act)[0], np.uint16)
        resb = np.full((1, h), _act_bits([float(res)], act)[0], np.uint16)
        gam = np.full((h,), _act_bits([1.0], act)[0], np.uint16)
        out = _run(part, resb, gam, 1e-6, act, act)
        got = act_bits_to_f64(out["residual_out"], act)
        assert np.all(got == float(want)), (act, p0, res, got[0, 0])


def test_fp32_partials_rank_order():
    # Same rule with fp32 partials: 2^24 + 1 + 1 - 2^24 -> 0 in rank order.
    part = np.array([2.0 ** 24, 1.0, 1.0, -2.0 ** 24], np.float32)[:, None, None]
    part = np.ascontiguousarray(np.broadcast_to(part, (4, 2, 8)))
    resb = np.full((2, 8), _act_bits([0.75], "bf16")[0], np.uint16)
    gam = np.full((8,), _act_bits([1.0], "bf16")[0], np.uint16)
    out = _run(part, resb, gam, 0.0, "f32", "bf16")
    assert np.all(act_bits_to_f64(out["residual_out"], "bf16") == 0.75)


# ---- exact arithmetic on tiny inputs -----------------------------------------------------

def _tiny_case(rng, n, t, h, pd, ad):
    """Partials k * 2^-4 (k small integers): every fp32 partial sum is exact, so the
    reduced value is the correctly rounded exact sum."""
    kmax = {"bf16": 127, "f16": 1023, "f32": 4095}[pd]
    k = rng.integers(-kmax, kmax + 1, size=(n, t, h)).astype(np.float64)
    pv = k * 2.0 ** -4
    if pd == "f32":
        pbits = pv.astype(np.float32)
    else:
        pbits = _act_bits(pv, pd)
    # residual k * 2^-6 with |k| <= 255: exact in both 16-bit types, and the sum with the
    # reduced value stays exact in fp32 (a multiple of 2^-6 below 2^14)
    rv = rng.integers(-255, 256, size=(t, h)).astype(np.float64) * 2.0 ** -6
    rbits = _act_bits(rv, ad)
    gv = rng.uniform(0.5, 1.5, size=h)
    gbits = numpy_f16_bits(gv) if ad == "f16" else torch_bf16_bits(gv.astype(np.float32))
    return pv, pbits, rbits, gbits


@pytest.mark.parametrize("pd,ad", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16"),
                                   ("f32", "f16")])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("h", [8, 16, 64, 264])
@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_exact_brute_force_tiny(pd, ad, n, h, eps):
    rng = np.random.default_rng(n * 1000 + h + (7 if pd == "f32" else 0))
    t = 5
    pv, pbits, rbits, gbits = _tiny_case(rng, n, t, h, pd, ad)
    out = _run(pbits, rbits, gbits, eps, pd, ad)
    # reduced value: exact sum (every fp32 partial sum is exact), rounded once
    exact_sum = pv.sum(axis=0)
    s_bits = exact_to_act_bits(exact_sum, ad)
    s = act_bits_to_f64(s_bits, ad)
    r_exact = s + act_bits_to_f64(rbits, ad)
    r_bits = exact_to_act_bits(r_exact, ad)
    assert np.array_equal(out["residual_out"], r_bits)
    # textbook RMSNorm of the rounded residual, fp64
    x = act_bits_to_f64(r_bits, ad)
    g = act_bits_to_f64(gbits, ad)
    y = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + np.float64(np.float32(eps))) * g
    got = act_bits_to_f64(out["norm_out"], ad)
    # the oracle's fp32 steps add at most a few 2^-24 relative before the final rounding
    bound = 0.5 * act_ulp(y, ad) + np.abs(y) * 2.0 ** -20
    assert np.all(np.abs(got - y) <= bound)


# ---- invariants ---------------------------------------------------------------------------

def _gen(name, tokens=None):
    w = workloads.WORKLOADS[name]
    if tokens is not None:
        w = w.with_tokens(tokens)
    p, r, g = workloads.generate(w, "cpu")
    return w, workloads.to_bits(p), workloads.to_bits(r), workloads.to_bits(g)


def test_n1_identity_is_rounded_exact_sum():
    rng = np.random.default_rng(5)
    for ad in ("bf16", "f16"):
        t, h = 6, 1024
        pv = rng.normal(0, 1, (1, t, h))
        pb = numpy_f16_bits(pv) if ad == "f16" else torch_bf16_bits(pv.astype(np.float32))
        rv = rng.normal(0, 1, (t, h))
        rb = numpy_f16_bits(rv) if ad == "f16" else torch_bf16_bits(rv.astype(np.float32))
        gb = _act_bits(np.ones(h), ad)
        out = _run(pb, rb, gb, 1e-6, ad, ad)
        exact = act_bits_to_f64(pb[0], ad) + act_bits_to_f64(rb, ad)
        # compare where the exact sum is an fp32 value (torch's cast is then one rounding);
        # numpy's fp64 -> f16 cast is a single rounding everywhere
        ok = exact.astype(np.float32).astype(np.float64) == exact
        assert ok.mean() > 0.99
        want = exact_to_act_bits(np.where(ok, exact, 0.0), ad)
        assert np.array_equal(out["residual_out"][ok], want[ok])


def test_gamma_one_gives_unit_rms():
    w, p, r, g = _gen("c0")
    g1 = _act_bits(np.ones(w.hidden), "bf16")
    out = _run(p, r, g1, 0.0, "bf16", "bf16")
    y = act_bits_to_f64(out["norm_out"], "bf16")
    rms = np.sqrt((y * y).mean(axis=1))
    # each output carries at most half a bf16 ulp (2^-9 relative) of rounding
    assert np.all(np.abs(rms - 1.0) < 2.0 ** -8)
    # and with eps the RMS is sqrt(m / (m + eps)) for the mean square m of the residual
    x = act_bits_to_f64(out["residual_out"], "bf16")
    m = (x * x).mean(axis=1)
    eps = 0.5
    out2 = _run(p, r, g1, eps, "bf16", "bf16")
    y2 = act_bits_to_f64(out2["norm_out"], "bf16")
    rms2 = np.sqrt((y2 * y2).mean(axis=1))
    assert np.all(np.abs(rms2 - np.sqrt(m / (m + np.float32(eps)))) < 2.0 ** -8)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_gamma_one_unit_rms_exactly_on_exact_rows(act):
    # Rows of +-1 and +-3 (40 and 24 of 64, random signs and places) times 2^k have the mean
    # square exactly 4 * 4^k, so with eps = 0 the scale is exactly 2^-(k+1) and every output
    # is +-0.5 or +-1.5, exact in bf16 and fp16: the output RMS must be 1 to the last bit
    # (the 1e-5 bar with no rounding allowance). A mean over H-1 (a 1.6% larger scale), a
    # root of the sum, or a mean of |x| instead of x^2 each move the outputs off +-0.5/+-1.5
    # by whole ulps.
    rng = np.random.default_rng(7)
    h, rows = 64, []
    for k in (-3, 0, 0, 4):
        mag = np.concatenate([np.ones(40), 3.0 * np.ones(24)])
        rng.shuffle(mag)
        rows.append(mag * rng.choice([-1.0, 1.0], size=h) * 2.0 ** k)
    x = np.array(rows)
    p = _act_bits(x[None], act)               # one shard, residual zero: r = x exactly
    r = _act_bits(np.zeros_like(x), act)
    g1 = _act_bits(np.ones(h), act)
    out = _run(p, r, g1, 0.0, act, act)
    assert np.array_equal(out["residual_out"], _act_bits(x, act))
    y = act_bits_to_f64(out["norm_out"], act)
    assert np.array_equal(np.abs(y) * 2.0, np.abs(x) / np.abs(x).min(axis=1, keepdims=True))
    rms = np.sqrt((y * y).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 1e-5) and np.all(rms == 1.0)


def test_power_of_two_scaling_leaves_output_unchanged():
    w, p, r, g = _gen("c0")
    base = _run(p, r, g, 0.0, "bf16", "bf16")
    for k in (-3, 5):
        f = np.float32(2.0 ** k)
        ps = torch_bf16_bits(act_bits_to_f64(p, "bf16").astype(np.float32) * f)
        rs = torch_bf16_bits(act_bits_to_f64(r, "bf16").astype(np.float32) * f)
        out = _run(ps, rs, g, 0.0, "bf16", "bf16")
        assert np.array_equal(out["norm_out"], base["norm_out"])
        assert np.array_equal(act_bits_to_f64(out["residual_out"], "bf16"),
                              act_bits_to_f64(base["residual_out"], "bf16") * float(f))


def test_channel_permutation_equivariance():
    w, p, r, g = _gen("c0")
    perm = np.random.default_rng(9).permutation(w.hidden)
    base = _run(p, r, g, w.eps, "bf16", "bf16")
    out = _run(np.ascontiguousarray(p[:, :, perm]), np.ascontiguousarray(r[:, perm]),
               np.ascontiguousarray(g[perm]), w.eps, "bf16", "bf16")
    assert np.array_equal(out["residual_out"], base["residual_out"][:, perm])
    assert ulp_diff16(out["norm_out"], base["norm_out"][:, perm]).max() <= 1


def test_thread_count_invariance():
    w, p, r, g = _gen("c1", tokens=24)
    outs = [_run(p, r, g, w.eps, "bf16", "bf16", quant="per_token", n_threads=k)
            for k in (1, 3, 8)]
    for o in outs[1:]:
        for key in ("residual_out", "norm_out", "quant_out", "scale_out"):
            assert np.array_equal(o[key], outs[0][key])


def test_in_place_residual_matches_out_of_place():
    w, p, r, g = _gen("c0")
    base = _run(p, r, g, w.eps, "bf16", "bf16")
    r2 = r.copy()
    out = _run(p, r2, g, w.eps, "bf16", "bf16", residual_out_array=r2)
    assert np.array_equal(r2, base["residual_out"])
    assert np.array_equal(out["norm_out"], base["norm_out"])


def test_output_subsets_agree():
    w, p, r, g = _gen("c0")
    full = _run(p, r, g, w.eps, "bf16", "bf16")
    only_r = _run(p, r, g, w.eps, "bf16", "bf16", norm_out=False)
    only_n = _run(p, r, g, w.eps, "bf16", "bf16", residual_out=False)
    assert np.array_equal(only_r["residual_out"], full["residual_out"])
    assert np.array_equal(only_n["norm_out"], full["norm_out"])
    assert "norm_out" not in only_r and "residual_out" not in only_n


def test_fp32_outlier_workload_shape_and_norm():
    w, p, r, g = _gen("c3", tokens=4)
    cols = workloads.outlier_channels(w).numpy()
    assert cols.size == 72
    assert np.abs(p[:, :, cols]).mean() > 50 * np.abs(np.delete(p, cols, axis=2)).mean()
    out = _run(p, r, g, w.eps, "f32", "bf16")
    x = act_bits_to_f64(out["residual_out"], "bf16")
    gg = act_bits_to_f64(g, "bf16")
    y = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + np.float64(np.float32(w.eps))) * gg
    got = act_bits_to_f64(out["norm_out"], "bf16")
    assert np.all(np.abs(got - y) <= 0.5 * act_ulp(y, "bf16") + np.abs(y) * 2.0 ** -20)
    # reduced value: fp32 rank-order sum of fp32 partials; within the error of N-1
    # fp32 additions of the exact sum, then rounded to bf16 and added to the residual
    exact = p.astype(np.float64).sum(axis=0)
    rr = exact + act_bits_to_f64(r, "bf16")
    tol = (act_ulp(exact, "bf16") + act_ulp(rr, "bf16")
           + np.abs(p).astype(np.float64).sum(axis=0) * 3 * 2.0 ** -24)
    assert np.all(np.abs(x - rr) <= tol)


# ---- fp8 copy ------------------------------------------------------------------------------

def test_per_token_amax_code_and_dequant_bound():
    w, p, r, g = _gen("c2", tokens=16)
    out = _run(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    y = act_bits_to_f64(out["norm_out"], "bf16")
    q, sc = out["quant_out"], out["scale_out"].astype(np.float64)
    amax = np.abs(y).max(axis=1)
    assert np.allclose(sc * 448.0, amax, rtol=2.0 ** -22, atol=0)
    # the element(s) of largest magnitude map to +-448
    for t in range(y.shape[0]):
        i = np.nonzero(np.abs(y[t]) == amax[t])[0]
        assert np.all((q[t, i] & 0x7F) == 0x7E)
    deq = e4m3_code_to_f64(q) * sc[:, None]
    sub = (q & 0x78) == 0
    err = np.abs(deq - y)
    assert np.all(err[~sub] <= np.abs(y[~sub]) * (2.0 ** -4 + 2.0 ** -20))
    assert np.all(err[sub] <= (2.0 ** -10 * (1 + 2.0 ** -20)) * np.broadcast_to(sc[:, None], y.shape)[sub])


def test_per_tensor_power_of_two_scale_is_exact_brute_force():
    w, p, r, g = _gen("c2", tokens=8)
    for k in (-2, 0, 3):
        out = _run(p, r, g, w.eps, "bf16", "bf16", quant="per_tensor", scale_in=2.0 ** k)
        y = act_bits_to_f64(out["norm_out"], "bf16")
        # y * 2^-k is exact, so the code is the brute-force nearest E4M3 value
        want = e4m3_brute(y * 2.0 ** -k).reshape(y.shape)
        assert np.array_equal(out["quant_out"], want)


def test_zero_scale_and_zero_row_give_zero_codes():
    h = 64
    part = np.zeros((2, 3, h), np.uint16)
    res = np.zeros((3, h), np.uint16)
    gam = _act_bits(np.ones(h), "bf16")
    out = _run(part, res, gam, 1e-6, "bf16", "bf16", quant="per_token")
    assert np.all(out["quant_out"] == 0) and np.all(out["scale_out"] == 0)
    assert np.all(ordinal16(out["norm_out"]) == 0)
    w, p, r, g = _gen("c0", tokens=2)
    out = _run(p, r, g, w.eps, "bf16", "bf16", quant="per_tensor", scale_in=0.0)
    assert np.all((out["quant_out"] & 0x7F) == 0)


def test_per_tensor_and_per_token_agree_when_scales_agree():
    w, p, r, g = _gen("c2", tokens=1)
    tok = _run(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    ten = _run(p, r, g, w.eps, "bf16", "bf16", quant="per_tensor",
               scale_in=float(tok["scale_out"][0]))
    assert np.array_equal(tok["quant_out"], ten["quant_out"])
    assert code_diff8(tok["quant_out"], tok["quant_out"]).max() == 0


def test_argument_errors():
    p = np.zeros((2, 1, 8), np.uint16)
    r = np.zeros((1, 8), np.uint16)
    g = np.zeros((8,), np.uint16)
    with pytest.raises(oracle.OracleError):
        _run(p, r, g, -1.0, "bf16", "bf16")
    with pytest.raises(oracle.OracleError):
        _run(p, r, g, 1e-6, "bf16", "bf16", residual_out=False, norm_out=False)
    L = oracle.lib()
    assert L.arfo_reduce_add_rmsnorm(None, 2, 1, 8, 0, 0, None, None, None, 0.0, None, 1) == 1
    assert L.arfo_reduce_add_rmsnorm(p.ctypes.data, 0, 1, 8, 0, 0, r.ctypes.data, r.ctypes.data,
                                     g.ctypes.data, 0.0, None, 1) == 2
    assert L.arfo_reduce_add_rmsnorm(p.ctypes.data, 2, 1, 8, 2, 2, r.ctypes.data, r.ctypes.data,
                                     g.ctypes.data, 0.0, None, 1) == 3
    # tokens == 0 is a valid empty call
    assert L.arfo_reduce_add_rmsnorm(p.ctypes.data, 2, 0, 8, 0, 0, r.ctypes.data, r.ctypes.data,
                                     g.ctypes.data, 0.0, None, 1) == 0


def test_generator_is_reproducible_and_has_the_stated_moments():
    w = workloads.WORKLOADS["c1"].with_tokens(32)
    a = workloads.generate(w, "cpu")
    b = workloads.generate(w, "cpu")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    p = a[0].float()
    assert abs(p.std().item() - 0.5) < 0.01 and abs(a[1].float().std().item() - 1.0) < 0.02
    gmin, gmax = a[2].float().min().item(), a[2].float().max().item()
    assert 0.5 <= gmin and gmax <= 1.5


# ---- special values (IEEE 754 propagation through the method's steps) -----------------------

def _special_case(value, act="bf16"):
    w = workloads.WORKLOADS["c0"].with_tokens(3)
    p, r, g = (workloads.to_bits(x) for x in workloads.generate(w, "cpu"))
    p = p.copy()
    p[1, 1, 5] = _act_bits([value], act)[0] if np.isfinite(value) else \
        (0x7FC0 if np.isnan(value) else (0x7F80 if value > 0 else 0xFF80))
    return w, p, r, g


def test_nan_partial_poisons_its_element_and_its_row_norm():
    w, p, r, g = _special_case(float("nan"))
    out = _run(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    x = act_bits_to_f64(out["residual_out"], "bf16")
    y = act_bits_to_f64(out["norm_out"], "bf16")
    assert np.isnan(x[1, 5]) and np.isnan(x).sum() == 1
    assert np.all(np.isnan(y[1])) and not np.any(np.isnan(y[[0, 2]]))
    # the per-token max skips NaN; every code of the row is a NaN code
    assert np.all((out["quant_out"][1] & 0x7F) == 0x7F)
    assert not np.isnan(out["scale_out"][1])


def test_infinite_partial_gives_zero_inverse_root():
    w, p, r, g = _special_case(float("inf"))
    out = _run(p, r, g, w.eps, "bf16", "bf16")
    x = act_bits_to_f64(out["residual_out"], "bf16")
    y = act_bits_to_f64(out["norm_out"], "bf16")
    assert x[1, 5] == np.inf
    # sum of squares is inf, so 1/sqrt(.) = 0: finite elements give +-0, the inf one NaN
    assert np.isnan(y[1, 5])
    finite = np.delete(y[1], 5)
    assert np.all(finite == 0.0)
    assert np.array_equal(np.signbit(finite), np.signbit(np.delete(x[1], 5)))


def test_negative_zeros_stay_negative():
    h = 64
    p = np.full((3, 2, h), 0x8000, np.uint16)
    r = np.full((2, h), 0x8000, np.uint16)
    g = _act_bits(np.ones(h), "bf16")
    out = _run(p, r, g, 1e-6, "bf16", "bf16", quant="per_token")
    assert np.all(out["residual_out"] == 0x8000)     # -0 + -0 = -0 at every step
    assert np.all(out["norm_out"] == 0x8000)         # (-0 * inv) * 1 = -0
    assert np.all(out["quant_out"] == 0x80) and np.all(out["scale_out"] == 0)
    # +0 residual: -0 + +0 = +0
    out = _run(p, np.zeros((2, h), np.uint16), g, 1e-6, "bf16", "bf16")
    assert np.all(out["residual_out"] == 0x0000)


def test_oracle_args_struct_follows_its_header():
    import ctypes
    import os
    import re
    hdr = os.path.join(os.path.dirname(oracle.__file__), "arf_oracle.h")
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    body = re.search(r"typedef struct arfo_args \{(.*?)\} arfo_args;", text, flags=re.S).group(1)
    fields = [l.strip().rstrip(";") for l in body.splitlines() if l.strip()]
    assert [f.split()[-1].lstrip("*") for f in fields] == [n for n, _ in oracle.Args._fields_]
    sizes = {"int32_t": 4, "int64_t": 8, "float": 4}
    for f, (n, ct) in zip(fields, oracle.Args._fields_):
        if "*" in f:
            assert ct is ctypes.c_void_p, n
        else:
            assert ctypes.sizeof(ct) == sizes[f.split()[0]], n
