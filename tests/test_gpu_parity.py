"""GPU parity: the HIP path (through the C ABI) against the oracle, element by element.

Tolerances (fixed here, per output):
  residual_out  bit-exact;
  norm_out      at most 1 ulp of the activation type (ordinal distance, +0 == -0);
  fp8 codes     at most 1 code (ordinal distance);
  scale_out     bit-exact in every row whose norm_out is bit-exact (both sides take
                fl32(amax / 448) of the same values); relative 2^-7 in a row whose outputs
                differ by the 1 ulp allowed.
Every element must pass. Output buffers are poisoned (0xFF) and followed by canary
bytes, so an element that is never written, or a write past the end, fails.
"""
import ctypes
import numpy as np
import pytest
import torch

import oracle
import shard_reduce_residual_amd as arf
import workloads
from helpers import code_diff8, e4m3_brute, ulp_diff16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 512
POISON, CANARY = 0xFF, 0x5A
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
THREADS = min(16, oracle.default_threads())


def say(msg):
    print("[case] " + msg, flush=True)


class Out:
    """An output tensor with a poisoned body and a canary tail."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.nbytes = n
        self.raw = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device=DEV)
        self.raw[n:] = CANARY
        self.t = self.raw[:n].view(dtype).view(shape)

    def canary_ok(self):
        return bool((self.raw[self.nbytes:] == CANARY).all().item())


def run_gpu(p, r, g, eps, act, *, res=True, norm=True, quant=None, scale=None,
            in_place=False, stream=None):
    """p, r, g: device tensors. Returns host numpy results (uint16 bits / uint8 / f32).
    ``stream``: a stream handle for the call (default: torch's current stream); the call
    then starts after a device synchronisation."""
    t, h = r.shape
    adt = TORCH[act]
    rin = r.clone() if in_place else r
    rout = None
    if in_place:
        rout_t = rin
    elif res:
        rout = Out((t, h), adt)
        rout_t = rout.t
    else:
        rout_t = None
    nout = Out((t, h), adt) if norm else None
    out = {}
    if stream is not None:
        torch.cuda.synchronize()
    if quant is None:
        arf.arf_reduce_add_rmsnorm(p, rin, g, eps, residual_out=rout_t,
                                   norm_out=nout.t if nout else None, stream=stream)
    else:
        q = Out((t, h), torch.uint8)
        sin = sout = None
        if quant == "per_tensor":
            sin = torch.tensor([scale], dtype=torch.float32, device=DEV)
            mode = arf.ARF_QUANT_PER_TENSOR
        else:
            sout = Out((t,), torch.float32)
            mode = arf.ARF_QUANT_PER_TOKEN
        if stream is not None:
            torch.cuda.synchronize()
        arf.arf_reduce_add_rmsnorm_quant(p, rin, g, eps, q.t, mode, scale_in=sin,
                                         scale_out=sout.t if sout else None,
                                         residual_out=rout_t,
                                         norm_out=nout.t if nout else None, stream=stream)
        torch.cuda.synchronize()
        assert q.canary_ok()
        out["quant_out"] = q.t.cpu().numpy()
        if sout is not None:
            assert sout.canary_ok()
            out["scale_out"] = sout.t.cpu().numpy()
    torch.cuda.synchronize()
    if rout_t is not None:
        if rout is not None:
            assert rout.canary_ok()
        out["residual_out"] = workloads.to_bits(rout_t)
    if nout is not None:
        assert nout.canary_ok()
        out["norm_out"] = workloads.to_bits(nout.t)
    return out


def run_oracle(p, r, g, eps, pd, act, **kw):
    return oracle.reduce_add_rmsnorm(workloads.to_bits(p), workloads.to_bits(r),
                                     workloads.to_bits(g), eps, partial_dtype=pd,
                                     act_dtype=act, n_threads=THREADS, **kw)


def compare(gpu, ref, label="", min_exact=0.999):
    stats = {}
    if "residual_out" in ref and "residual_out" in gpu:
        bad = np.nonzero(gpu["residual_out"] != ref["residual_out"])
        assert bad[0].size == 0, "%s residual_out differs at %s" % (label, list(zip(*bad))[:5])
    if "norm_out" in ref and "norm_out" in gpu:
        d = ulp_diff16(gpu["norm_out"], ref["norm_out"])
        stats["norm_exact"] = float((d == 0).mean())
        assert d.max() <= 1, "%s norm_out differs by %d ulp" % (label, d.max())
        assert stats["norm_exact"] >= min_exact, (label, stats)
    if "quant_out" in ref:
        d = code_diff8(gpu["quant_out"], ref["quant_out"])
        stats["fp8_exact"] = float((d == 0).mean())
        assert d.max() <= 1, "%s fp8 codes differ by %d" % (label, d.max())
    if "scale_out" in ref:
        # both sides compute fl32(amax / 448) from the cast outputs: where a row's norm_out
        # is bit-identical to the oracle's, its scale must be too (NaN where the oracle has
        # NaN); in a row whose outputs differ by the 1 ulp allowed, the row maximum may
        # differ by as much, and the scale by 2^-7 relative
        gs = np.asarray(gpu["scale_out"], dtype=np.float32)
        rs = np.asarray(ref["scale_out"], dtype=np.float32)
        same = (np.isnan(gs) & np.isnan(rs)) | (gs.view(np.uint32) == rs.view(np.uint32))
        if "norm_out" in ref and "norm_out" in gpu and gs.size:
            rows_equal = np.all(np.asarray(gpu["norm_out"]) == np.asarray(ref["norm_out"]),
                                axis=tuple(range(1, np.asarray(ref["norm_out"]).ndim)))
        else:
            rows_equal = np.zeros(gs.shape, bool)
        assert same[rows_equal].all(), "%s scale_out differs at %s" % (
            label, np.nonzero(rows_equal & ~same)[0][:5])
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.abs(gs.astype(np.float64) / rs - 1.0)
        rel = np.where(rs == 0, np.abs(gs), rel)
        rel = np.where(same, 0.0, rel)
        assert rel.max(initial=0.0) <= 2.0 ** -7, (label, rel.max())
        stats["scale_exact"] = float(same.mean()) if same.size else 1.0
    return stats


def upload(w):
    p, r, g = workloads.generate(w, "cpu")
    return (p, r, g), (p.to(DEV), r.to(DEV), g.to(DEV))


def test_inputs_are_the_same_on_the_gpu_and_the_cpu():
    # the counter-based generator gives the same bits on either device: c0..c3 whole, and
    # the largest workload (generated whole on the GPU by the benchmark and the tests) in
    # its first and last 64 rows of every shard, from the CPU row generator
    for key in ("c0", "c1", "c2", "c3"):
        w = workloads.WORKLOADS[key]
        say("generator %s cpu vs gpu" % w.name)
        for a, b in zip(workloads.generate(w, "cpu"), workloads.generate(w, DEV)):
            assert torch.equal(a, b.cpu()), w.name
    w = workloads.WORKLOADS["c4"]
    p, r, g = workloads.generate(w, DEV)
    for b in (0, w.tokens - 64):
        say("generator %s rows %d..%d cpu vs gpu" % (w.name, b, b + 64))
        pc, rc, gc = workloads.generate_rows(w, b, 64, "cpu")
        assert torch.equal(pc, p[:, b:b + 64].cpu()), b
        assert torch.equal(rc, r[b:b + 64].cpu()), b
        assert torch.equal(gc, g.cpu())
    del p, r

# ---- the five workloads --------------------------------------------------------------------

@pytest.mark.parametrize("key", ["c0", "c1", "c2", "c3"])
def test_workload_parity_full(key):
    w = workloads.WORKLOADS[key]
    say("workload %s full compare" % w.name)
    (p, r, g), (pd_, rd, gd) = upload(w)
    scale = None
    if w.quant == "per_tensor":
        # the per-tensor scale is max|y| / 448 of the oracle's own normalised output
        y = oracle.act_to_f32(run_oracle(p, r, g, w.eps, w.partial_dtype, w.act_dtype)["norm_out"],
                              w.act_dtype)
        scale = float(np.float32(np.abs(y).max()) / np.float32(448.0))
    ref = run_oracle(p, r, g, w.eps, w.partial_dtype, w.act_dtype, quant=w.quant,
                     scale_in=scale)
    got = run_gpu(pd_, rd, gd, w.eps, w.act_dtype, quant=w.quant, scale=scale)
    stats = compare(got, ref, w.name)
    print(w.name, stats)


@pytest.mark.parametrize("path", [0, 2, 3])
def test_workload_c4_full_size_every_row(path):
    # the largest workload at full size, in the launch configuration the benchmark times
    # (path 0: the plan, rows claimed in start order), with rows by workgroup index (path
    # 2), and with the held-row kernel forced (eight batches of four rows per workgroup):
    # every row against the oracle, 1024 rows at a time
    w = workloads.WORKLOADS["c4"]
    say("workload %s full size, every row, path %d" % (w.name, path))
    p, r, g = workloads.generate(w, DEV)
    t, h = w.tokens, w.hidden
    rout = torch.empty((t, h), dtype=torch.bfloat16, device=DEV)
    nout = torch.empty((t, h), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((t, h), dtype=torch.uint8, device=DEV)
    sc = torch.empty((t,), dtype=torch.float32, device=DEV)
    try:
        arf.arf_set_path_override(path)
        arf.arf_reduce_add_rmsnorm_quant(p, r, g, w.eps, q, arf.ARF_QUANT_PER_TOKEN, scale_out=sc,
                                         residual_out=rout, norm_out=nout)
        torch.cuda.synchronize()
    finally:
        arf.arf_set_path_override(0)
    exact = []
    for b in range(0, t, 1024):
        e = min(t, b + 1024)
        say("c4 rows %d..%d" % (b, e))
        ref = run_oracle(p[:, b:e].contiguous(), r[b:e].contiguous(), g, w.eps, "bf16", "bf16",
                         quant="per_token")
        got = {"residual_out": workloads.to_bits(rout[b:e]),
               "norm_out": workloads.to_bits(nout[b:e]),
               "quant_out": q[b:e].cpu().numpy(), "scale_out": sc[b:e].cpu().numpy()}
        exact.append(compare(got, ref, "%s rows %d..%d" % (w.name, b, e)))
    print(w.name, exact[0], exact[-1])
    # properties over every row: the scale is max|y|/448 of the row, and the element(s)
    # of largest magnitude carry the code 448
    y = nout.float().abs()
    amax = y.amax(dim=1)
    assert torch.allclose(sc.double() * 448.0, amax.double(), rtol=2.0 ** -22, atol=0)
    top = (y == amax[:, None])
    assert bool(((q[top] & 0x7F) == 0x7E).all())
    del p, r, rout, nout, q


# ---- sizes, shapes, types and paths --------------------------------------------------------

def _case(n, t, h, pd, ad, seed, quant=None, eps=1e-6, std=1.0):
    w = workloads.Workload("sweep", n, t, h, pd, ad, std, 1.0, eps, quant, seed)
    return w


SWEEP = [  # (n, t, h)
    (1, 3, 8), (2, 5, 16), (3, 17, 64), (16, 2, 264), (7, 9, 1024), (8, 33, 2048),
    (5, 4, 4096), (4, 6, 7168), (8, 3, 8192), (9, 2, 16384), (2, 1, 32768), (1, 2, 65536),
    (16, 2, 65536), (12, 3, 7176), (6, 65, 520),
]


@pytest.mark.parametrize("pd,ad", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16"),
                                   ("f32", "f16")])
def test_sweep_shapes_auto_path(pd, ad):
    for i, (n, t, h) in enumerate(SWEEP):
        w = _case(n, t, h, pd, ad, 100 + i, quant="per_token" if i % 2 else None)
        say("sweep auto n=%d t=%d h=%d %s/%s quant=%s" % (n, t, h, pd, ad, w.quant))
        (p, r, g), (pd_, rd, gd) = upload(w)
        ref = run_oracle(p, r, g, w.eps, pd, ad, quant=w.quant)
        got = run_gpu(pd_, rd, gd, w.eps, ad, quant=w.quant)
        compare(got, ref, "n=%d t=%d h=%d" % (n, t, h), min_exact=0.99)


XN = (1, 2, 3, 4, 7, 8, 16)
XT = (1, 2, 3, 17, 64)
XH = (8, 16, 64, 264, 1024, 2048, 4096, 7168, 8192, 16384)


@pytest.mark.parametrize("pd,ad", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16"),
                                   ("f32", "f16")])
def test_cross_product_sweep_both_paths(pd, ad):
    # N x T x H over small token counts, per-token fp8 on every other case, each case on
    # the planned geometry, again with the other one-row path forced (one row per wavefront
    # only where a wavefront covers the row), with the held-row kernel forced, and with
    # every row claimed from the stream's counter (calls of many sizes one after another on
    # one stream: each must find the counter back at 0); every fourth case in place
    for n in XN:
        for t in XT:
            for h in XH:
                quant = "per_token" if (n + t) % 2 else None
                w = _case(n, t, h, pd, ad, 7000 + 100 * n + t, quant=quant)
                (p, r, g), (pd_, rd, gd) = upload(w)
                ref = run_oracle(p, r, g, w.eps, pd, ad, quant=quant)
                auto = arf.arf_get_plan(n, t, h, {"bf16": 0, "f16": 1, "f32": 2}[pd])["path"]
                other = 2 if auto == 1 else (1 if h <= 4096 else None)
                in_place = (n + t + h // 8) % 4 == 0
                for forced in (0, other, 3, 4):
                    if forced is None or forced == auto:
                        continue
                    say("cross n=%d t=%d h=%d %s/%s quant=%s path=%s in_place=%s"
                        % (n, t, h, pd, ad, quant, forced or "auto", in_place))
                    try:
                        arf.arf_set_path_override(forced)
                        got = run_gpu(pd_, rd, gd, w.eps, ad, quant=quant, in_place=in_place)
                    finally:
                        arf.arf_set_path_override(0)
                    compare(got, ref, "n=%d t=%d h=%d path=%s" % (n, t, h, forced or "auto"),
                            min_exact=0.99)

def _geometries(h, pd="bf16"):
    hc = h // 8
    out = []
    for c in (1, 2, 4, 8):
        if 64 * c >= hc:
            out.append((1, 4, c))
        for wv in (4, 8, 16):
            if wv * 64 * c >= hc:
                out.append((2, wv, c))
        if 256 * c >= hc:
            out.append((3, 4, c))   # held rows: 4 wavefronts
        if pd != "f32" and c <= 4 and 512 * c >= hc:
            out.append((3, 8, c))   # held rows: 8 wavefronts (16-bit partials)
        for wv in (4, 8, 16):
            if wv * 64 * c >= hc:
                out.append((4, wv, c))   # one row per workgroup, every row claimed
    return out


@pytest.mark.parametrize("h", [264, 1024, 4096, 7168])
def test_every_geometry_matches_the_oracle(h):
    w = _case(8, 7, h, "bf16", "bf16", 7 + h, quant="per_token")
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    try:
        for path, wv, c in _geometries(h):
            say("geometry h=%d path=%d waves=%d chunks=%d" % (h, path, wv, c))
            arf.arf_set_path_override(path, wv if path != 1 else 0, c)
            got = run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_token")
            compare(got, ref, "h=%d path=%d w=%d c=%d" % (h, path, wv, c), min_exact=0.99)
    finally:
        arf.arf_set_path_override(0)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16])
def test_every_shard_count(n):
    w = _case(n, 4, 2048, "bf16", "bf16", 300 + n)
    say("shards n=%d" % n)
    (p, r, g), (pd_, rd, gd) = upload(w)
    compare(run_gpu(pd_, rd, gd, w.eps, "bf16"), run_oracle(p, r, g, w.eps, "bf16", "bf16"))


@pytest.mark.parametrize("pd,c", [("f32", 2), ("f32", 4), ("f32", 8), ("bf16", 8)])
def test_eight_wave_geometry_every_shard_count(pd, c):
    # the 8-wave geometry keeps 1 to 3 shards in flight depending on its load registers
    # (16-byte pieces per lane: C for 16-bit partials, 2C for fp32); every shard count
    # 1..16 runs through its prefetch ring, on a ragged row that fills all C chunks
    h = 8 * 64 * 8 * c - 24
    try:
        arf.arf_set_path_override(2, 8, c)
        for n in range(1, 17):
            w = _case(n, 3, h, pd, "bf16", 500 + 17 * c + n, quant="per_token" if n % 2 else None)
            say("8-wave geometry %s c=%d n=%d h=%d" % (pd, c, n, h))
            (p, r, g), (pd_, rd, gd) = upload(w)
            ref = run_oracle(p, r, g, w.eps, pd, "bf16", quant=w.quant)
            got = run_gpu(pd_, rd, gd, w.eps, "bf16", quant=w.quant)
            compare(got, ref, "%s c=%d n=%d" % (pd, c, n), min_exact=0.99)
    finally:
        arf.arf_set_path_override(0)


def test_output_subsets_and_in_place():
    w = _case(4, 9, 4096, "bf16", "bf16", 11)
    (p, r, g), (pd_, rd, gd) = upload(w)
    full = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    for kw in (dict(res=True, norm=False), dict(res=False, norm=True),
               dict(in_place=True), dict(res=False, norm=False, quant="per_token"),
               dict(in_place=True, norm=False, quant="per_token")):
        say("subset %s" % kw)
        got = run_gpu(pd_, rd, gd, w.eps, "bf16", **kw)
        ref = {k: v for k, v in full.items() if k in got}
        if "quant_out" not in got:
            ref.pop("scale_out", None)
        compare(got, ref, str(kw))
    # in place really overwrote the residual, and the input partials are untouched
    rin = rd.clone()
    arf.arf_reduce_add_rmsnorm(pd_, rin, gd, w.eps, residual_out=rin)
    torch.cuda.synchronize()
    assert np.array_equal(workloads.to_bits(rin), full["residual_out"])
    assert torch.equal(pd_.cpu(), p)


def test_per_tensor_scales_and_zero_rows():
    w = _case(2, 6, 1024, "bf16", "bf16", 12, quant="per_tensor")
    (p, r, g), (pd_, rd, gd) = upload(w)
    for scale in (2.0 ** -3, 0.0123, 1.0, 0.0, -1.0):
        say("per-tensor scale %g" % scale)
        ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_tensor", scale_in=scale)
        compare(run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_tensor", scale=scale), ref)
    say("all-zero rows, per-token")
    z = torch.zeros_like(pd_)
    zr = torch.zeros_like(rd)
    got = run_gpu(z, zr, gd, w.eps, "bf16", quant="per_token")
    assert np.all(got["quant_out"] == 0) and np.all(got["scale_out"] == 0)
    assert np.all((got["norm_out"] & 0x7FFF) == 0) and np.all(got["residual_out"] == 0)


def test_eps_values_and_outliers():
    for eps in (0.0, 1e-6, 0.5):
        w = workloads.Workload("out", 4, 5, 7168, "f32", "bf16", 1.0, 1.0, eps, None, 21,
                               outlier_frac=0.01, outlier_scale=100.0)
        say("fp32 partials with outliers eps=%g" % eps)
        (p, r, g), (pd_, rd, gd) = upload(w)
        compare(run_gpu(pd_, rd, gd, eps, "bf16"), run_oracle(p, r, g, eps, "f32", "bf16"))


def test_rank_order_vector_on_gpu():
    # 2^24 + 1 + 1 - 2^24 in rank order is 0 (a pairwise tree gives 1, the exact sum 2)
    say("rank-order vector")
    h = 64
    vals = torch.tensor([2.0 ** 24, 1.0, 1.0, -2.0 ** 24])
    p = vals[:, None, None].expand(4, 3, h).contiguous().to(torch.bfloat16).to(DEV)
    r = torch.full((3, h), 0.5, dtype=torch.bfloat16, device=DEV)
    g = torch.ones((h,), dtype=torch.bfloat16, device=DEV)
    got = run_gpu(p, r, g, 1e-6, "bf16")
    assert np.all(got["residual_out"] == 0x3F00)   # 0.5


def test_binding_rejects_bad_tensors_and_launches_nothing():
    say("binding argument checks")
    w = _case(2, 4, 64, "bf16", "bf16", 5)
    p, r, g = workloads.generate(w, DEV)
    nout = Out((4, 64), torch.bfloat16)
    bad = [
        dict(residual_in=r.cpu()),                                          # host tensor
        dict(norm_out=torch.empty((3, 64), dtype=torch.bfloat16, device=DEV)),   # short
        dict(residual_out=torch.empty((4, 64), dtype=torch.float32, device=DEV)),  # dtype
        dict(gamma=g[:32]),                                                 # short gamma
    ]
    for kw in bad:
        args = dict(residual_in=r, gamma=g, norm_out=nout.t)
        args.update(kw)
        with pytest.raises((ValueError, TypeError)):
            arf.arf_reduce_add_rmsnorm(p, args["residual_in"], args["gamma"], 1e-6,
                                       residual_out=args.get("residual_out"),
                                       norm_out=args["norm_out"])
    q = torch.empty((4, 64), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):   # per-token scales for 3 of 4 rows
        arf.arf_reduce_add_rmsnorm_quant(p, r, g, 1e-6, q, arf.ARF_QUANT_PER_TOKEN,
                                         scale_out=torch.empty(3, device=DEV), norm_out=nout.t)
    with pytest.raises(ValueError):   # MXFP4 codes sized for fp8
        arf.arf_fused_epilogue(p, r, g, 1e-6, norm_out=nout.t, quant_out=q,
                               mode=arf.ARF_QUANT_MXFP4,
                               scale_out=torch.empty((4, 2), dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert bool((nout.raw == POISON)[: nout.nbytes].all()) and nout.canary_ok()


def test_empty_call_writes_nothing():
    say("tokens == 0")
    p = torch.empty((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    r = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.ones((64,), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    arf.arf_reduce_add_rmsnorm(p, r, g, 1e-6, residual_out=o, norm_out=None)
    torch.cuda.synchronize()


def test_repeat_runs_are_bit_identical():
    w = workloads.WORKLOADS["c1"]
    say("determinism %s" % w.name)
    (p, r, g), (pd_, rd, gd) = upload(w)
    a = run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_token")
    b = run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_token")
    for k in a:
        assert np.array_equal(a[k], b[k])



@pytest.mark.parametrize("path", [0, 4])
def test_concurrent_calls_from_two_threads_on_two_streams(path):
    # two host threads enqueue calls with different shapes, types and modes on their own
    # streams at the same time; with path 4 every row is claimed, each stream from its own
    # counter while the other stream's launches run
    import threading

    cases = [_case(8, 128, 4096, "bf16", "bf16", 601),
             _case(4, 96, 7168, "f32", "bf16", 602, quant="per_token")]
    say("two threads, two streams")
    work = []
    for w in cases:
        (p, r, g), (pd_, rd, gd) = upload(w)
        ref = run_oracle(p, r, g, w.eps, w.partial_dtype, w.act_dtype, quant=w.quant)
        t, h = w.tokens, w.hidden
        outs = {"residual_out": Out((t, h), torch.bfloat16), "norm_out": Out((t, h), torch.bfloat16)}
        if w.quant:
            outs["quant_out"] = Out((t, h), torch.uint8)
            outs["scale_out"] = Out((t,), torch.float32)
        work.append((w, (pd_, rd, gd), outs, ref, torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []

    def enqueue(w, ins, outs, stream):
        try:
            pd_, rd, gd = ins
            for _ in range(25):
                if w.quant:
                    arf.arf_reduce_add_rmsnorm_quant(
                        pd_, rd, gd, w.eps, outs["quant_out"].t, arf.ARF_QUANT_PER_TOKEN,
                        scale_out=outs["scale_out"].t, residual_out=outs["residual_out"].t,
                        norm_out=outs["norm_out"].t, stream=stream)
                else:
                    arf.arf_reduce_add_rmsnorm(pd_, rd, gd, w.eps,
                                               residual_out=outs["residual_out"].t,
                                               norm_out=outs["norm_out"].t, stream=stream)
        except Exception as e:   # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=enqueue, args=(w, ins, outs, st))
               for w, ins, outs, _, st in work]
    try:
        arf.arf_set_path_override(path)
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        torch.cuda.synchronize()
    finally:
        arf.arf_set_path_override(0)
    assert not errors, errors
    for w, _, outs, ref, _ in work:
        got = {}
        for k, o in outs.items():
            assert o.canary_ok(), (w.name, k)
            got[k] = o.t.cpu().numpy() if k in ("quant_out", "scale_out") else workloads.to_bits(o.t)
        compare(got, ref, w.name)

# ---- the quantiser's conversion and the copy probe -----------------------------------------

def test_e4m3_conversion_matches_the_oracle():
    say("e4m3 encoder")
    from helpers import e4m3_values
    vals = e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [456.0, 464.0, 472.0, 480.0, 1e4]]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(np.inf))])
    rng = np.random.default_rng(3)
    pts = np.concatenate([pts, np.exp2(rng.uniform(-16, 12, 1 << 20)).astype(np.float32)])
    pts = np.concatenate([pts, -pts, rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64)
                          .astype(np.uint32).view(np.float32),
                          np.array([np.inf, -np.inf, 0.0, -0.0, np.nan], np.float32)])
    x = torch.from_numpy(pts).to(DEV)
    out = torch.empty(x.numel(), dtype=torch.uint8, device=DEV)
    arf.arf_e4m3_encode(x, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.f32_to_e4m3(pts)
    nan = np.isnan(pts)
    bad = np.nonzero(got[~nan] != want[~nan])[0]
    assert bad.size == 0, [(float(pts[~nan][i]), hex(got[~nan][i]), hex(want[~nan][i]))
                           for i in bad[:10]]
    assert np.all((got[nan] & 0x7F) == 0x7F)
    # odd length: the tail is converted and nothing past it is written
    y = torch.from_numpy(pts[:1001]).to(DEV)
    o2 = torch.full((1001 + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    arf.arf_e4m3_encode(y, o2[:1001])
    torch.cuda.synchronize()
    o2 = o2.cpu().numpy()
    assert np.array_equal(o2[:1001][~nan[:1001]], want[:1001][~nan[:1001]])
    assert np.all(o2[1001:] == 0x5A)
    assert np.array_equal(e4m3_brute(pts[:4096]), want[:4096])


def _e2m1_gpu(x):
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    out = torch.empty(xd.numel(), dtype=torch.uint8, device=DEV)
    arf.arf_e2m1_encode(xd, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_e2m1_conversion_matches_the_oracle():
    # the MXFP4 store's element conversion (gfx950's packed fp32 -> fp4 instruction) on
    # every fp32 value of magnitude 2^-4 to 8, both signs: every rounding boundary of E2M1,
    # its ties and the saturation at 6; then zeros, subnormals, infinities, NaN (with its
    # sign) and random patterns of every magnitude
    say("e2m1 encoder")
    mant = np.arange(1 << 23, dtype=np.uint32)
    for e in range(123, 130):
        for sign in (0, 0x80000000):
            x = (mant | np.uint32((e << 23) | sign)).view(np.float32)
            got, want = _e2m1_gpu(x), oracle.f32_to_e2m1(x)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), int(got[i]), int(want[i]))
                                   for i in bad[:10]]
    rng = np.random.default_rng(4)
    x = np.concatenate([
        rng.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32),
        rng.integers(0, 1 << 23, 1 << 16, dtype=np.uint32).view(np.float32),   # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 6.0, -6.0, 1e30, -1e30],
                 np.float32)])
    assert np.array_equal(_e2m1_gpu(x), oracle.f32_to_e2m1(x))
    # odd length: the tail is converted and nothing past it is written
    y = torch.from_numpy(x[:1001]).to(DEV)
    o2 = torch.full((1001 + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    arf.arf_e2m1_encode(y, o2[:1001])
    torch.cuda.synchronize()
    o2 = o2.cpu().numpy()
    assert np.array_equal(o2[:1001], oracle.f32_to_e2m1(x[:1001])) and np.all(o2[1001:] == 0x5A)

def test_stream_copy_is_exact():
    for nbytes in (16, 4096 + 48, 3 * 32768 + 16, 64 << 20):
        say("stream copy %d bytes" % nbytes)
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
        dst = torch.full((nbytes + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        arf.arf_stream_copy(dst, src, nbytes)
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes], src)
        assert bool((dst[nbytes:] == CANARY).all())


# ---- accumulation in the partial type, row ranges, reduce-only ----------------------------

@pytest.mark.parametrize("pd,ad", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16")])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_partial_accumulation_parity(pd, ad, n):
    w = _case(n, 9, 2056, pd, ad, 500 + n, quant="per_token", std=4.0)
    say("partial accumulation n=%d %s/%s" % (n, pd, ad))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, pd, ad, quant="per_token", accumulate="partial")
    t, h = r.shape
    rout, nout = Out((t, h), TORCH[ad]), Out((t, h), TORCH[ad])
    q, sc = Out((t, h), torch.uint8), Out((t,), torch.float32)
    arf.arf_fused_epilogue(pd_, rd, gd, w.eps, residual_out=rout.t, norm_out=nout.t,
                           quant_out=q.t, scale_out=sc.t, accumulate=arf.ARF_ACC_PARTIAL)
    torch.cuda.synchronize()
    assert all(o.canary_ok() for o in (rout, nout, q, sc))
    got = {"residual_out": workloads.to_bits(rout.t), "norm_out": workloads.to_bits(nout.t),
           "quant_out": q.t.cpu().numpy(), "scale_out": sc.t.cpu().numpy()}
    compare(got, ref, "partial acc n=%d" % n)
    if pd != "f32" and n >= 8:   # the two branches really differ here
        ref32 = run_oracle(p, r, g, w.eps, pd, ad)
        assert not np.array_equal(ref32["residual_out"], ref["residual_out"])


def test_partial_accumulation_golden_on_gpu():
    from helpers import read_golden, exact_to_act_bits, act_bits_to_f64
    for act, acc, *vals in read_golden("partial_accumulation.txt"):
        say("golden partial accumulation %s %s %s" % (act, acc, vals))
        h = 64
        pv = torch.tensor([float(v) for v in vals[:4]], dtype=torch.float64)
        p = pv[:, None, None].expand(4, 2, h).contiguous().to(TORCH[act]).to(DEV)
        zero = torch.zeros((2, h), dtype=TORCH[act], device=DEV)
        g = torch.ones((h,), dtype=TORCH[act], device=DEV)
        out = torch.empty((2, h), dtype=TORCH[act], device=DEV)
        arf.arf_fused_epilogue(p, zero, g, 1e-6, residual_out=out,
                               accumulate=arf.ARF_ACC_PARTIAL if acc == "partial" else arf.ARF_ACC_F32)
        sums = torch.empty((2, h), dtype=TORCH[act], device=DEV)
        arf.arf_reduce_rows(p, sums, accumulate=arf.ARF_ACC_PARTIAL if acc == "partial" else arf.ARF_ACC_F32)
        torch.cuda.synchronize()
        assert torch.all(out.double() == float(vals[4])) and torch.all(sums.double() == float(vals[4]))


@pytest.mark.parametrize("path", [0, 3, 4])
@pytest.mark.parametrize("begin,count", [(0, 7), (5, 11), (13, -1), (40, 1), (0, -1), (20, 0)])
def test_row_ranges(begin, count, path):
    w = _case(8, 41, 4096, "bf16", "bf16", 600, quant="per_token")
    say("row range %d %d path %d" % (begin, count, path))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token", rows=(begin, count),
                     out_init=POISON)
    t, h = r.shape
    rout, nout = Out((t, h), torch.bfloat16), Out((t, h), torch.bfloat16)
    q, sc = Out((t, h), torch.uint8), Out((t,), torch.float32)
    try:
        arf.arf_set_path_override(path)
        arf.arf_fused_epilogue(pd_, rd, gd, w.eps, residual_out=rout.t, norm_out=nout.t,
                               quant_out=q.t, scale_out=sc.t, row_begin=begin, row_count=count)
        torch.cuda.synchronize()
    finally:
        arf.arf_set_path_override(0)
    assert all(o.canary_ok() for o in (rout, nout, q, sc))
    end = t if count < 0 else begin + count
    got = {"residual_out": workloads.to_bits(rout.t), "norm_out": workloads.to_bits(nout.t),
           "quant_out": q.t.cpu().numpy(), "scale_out": sc.t.cpu().numpy()}
    for k in got:   # rows outside the range were never written (still the poison bytes)
        outside = np.concatenate([got[k][:begin].ravel().view(np.uint8),
                                  got[k][end:].ravel().view(np.uint8)])
        assert np.all(outside == POISON), k
    inside = {k: v[begin:end] for k, v in got.items()}
    want = {k: v[begin:end] for k, v in ref.items()}
    if end > begin:
        compare(inside, want, "rows %d..%d" % (begin, end))


@pytest.mark.parametrize("pd,ad", [("bf16", "bf16"), ("f32", "f16")])
def test_reduce_rows_and_twoshot_composition(pd, ad):
    n, t, h = 8, 37, 7168
    w = _case(n, t, h, pd, ad, 700, quant="per_token")
    say("reduce rows / twoshot %s/%s" % (pd, ad))
    (p, r, g), (pd_, rd, gd) = upload(w)
    gathered = Out((t, h), TORCH[ad])
    for rank in range(n):   # the page's launcher: t // n rows each, the first t % n one more
        cnt = t // n + (1 if rank < t % n else 0)
        beg = rank * (t // n) + min(rank, t % n)
        arf.arf_reduce_rows(pd_, gathered.t, row_begin=beg, row_count=cnt)
    torch.cuda.synchronize()
    assert gathered.canary_ok()
    sums = oracle.reduce_rows(workloads.to_bits(p), partial_dtype=pd, act_dtype=ad)
    assert np.array_equal(workloads.to_bits(gathered.t), sums)
    # epilogue over the gathered values with one "shard" == the oneshot result
    two = run_gpu(gathered.t.view(1, t, h), rd, gd, w.eps, ad, quant="per_token")
    one = run_gpu(pd_, rd, gd, w.eps, ad, quant="per_token")
    for k in one:
        assert np.array_equal(two[k], one[k]), k
    compare(one, run_oracle(p, r, g, w.eps, pd, ad, quant="per_token"), "oneshot")



def test_reduce_rows_with_claimed_rows():
    # a reduce-only row range large enough for the plan to claim its rows (2100 rows of
    # 8 x 16384 bf16), twice on one stream, against the oracle; rows outside keep their poison
    n, t, h = 8, 4096, 16384
    beg, cnt = 1000, 2100
    w = _case(n, t, h, "bf16", "bf16", 701)
    assert arf.arf_get_plan(n, cnt, h, 0)["path"] == 4
    say("reduce rows with claimed rows")
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = oracle.reduce_rows(workloads.to_bits(p), partial_dtype="bf16", act_dtype="bf16",
                             rows=(beg, cnt), out_init=POISON, n_threads=THREADS)
    for k in range(2):
        out = Out((t, h), torch.bfloat16)
        arf.arf_reduce_rows(pd_, out.t, row_begin=beg, row_count=cnt)
        torch.cuda.synchronize()
        assert out.canary_ok()
        assert np.array_equal(workloads.to_bits(out.t), ref), k

# ---- OCP MXFP4 copy ------------------------------------------------------------------------

def _ord4(c):
    c = np.asarray(c, dtype=np.int32)
    return np.where(c & 8, -(c & 7), c)


def run_gpu_mx(p, r, g, eps, act):
    from helpers import unpack_fp4
    t, h = r.shape
    rout, nout = Out((t, h), TORCH[act]), Out((t, h), TORCH[act])
    q, sc = Out((t, h // 2), torch.uint8), Out((t, h // 32), torch.uint8)
    arf.arf_fused_epilogue(p, r, g, eps, residual_out=rout.t, norm_out=nout.t, quant_out=q.t,
                           mode=arf.ARF_QUANT_MXFP4, scale_out=sc.t)
    torch.cuda.synchronize()
    assert all(o.canary_ok() for o in (rout, nout, q, sc))
    return {"residual_out": workloads.to_bits(rout.t), "norm_out": workloads.to_bits(nout.t),
            "codes": unpack_fp4(q.t.cpu().numpy()), "scales": sc.t.cpu().numpy()}


def compare_mx(got, ref, label=""):
    from helpers import unpack_fp4
    compare({k: got[k] for k in ("residual_out", "norm_out")},
            {k: ref[k] for k in ("residual_out", "norm_out")}, label)
    assert np.array_equal(got["scales"], ref["scale_out"]), label
    d = np.abs(_ord4(got["codes"]) - _ord4(unpack_fp4(ref["quant_out"])))
    assert d.max() <= 1, label
    return float((d == 0).mean())


@pytest.mark.parametrize("pd,ad", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16"),
                                   ("f32", "f16")])
def test_mxfp4_parity(pd, ad):
    for n, t, h in ((1, 3, 32), (2, 5, 1024), (8, 17, 4096), (4, 9, 7168), (3, 2, 16384)):
        w = _case(n, t, h, pd, ad, 800 + h + n, std=2.0)
        say("mxfp4 n=%d t=%d h=%d %s/%s" % (n, t, h, pd, ad))
        (p, r, g), (pd_, rd, gd) = upload(w)
        ref = run_oracle(p, r, g, w.eps, pd, ad, quant="mxfp4")
        exact = compare_mx(run_gpu_mx(pd_, rd, gd, w.eps, ad), ref, "h=%d" % h)
        assert exact >= 0.999


@pytest.mark.parametrize("pd", ["bf16", "f32"])
def test_mxfp4_every_geometry(pd):
    h = 7168
    w = _case(8, 6, h, pd, "bf16", 900, std=3.0)
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, pd, "bf16", quant="mxfp4")
    try:
        for path, wv, c in _geometries(h, pd):
            say("mxfp4 geometry %s path=%d waves=%d chunks=%d" % (pd, path, wv, c))
            arf.arf_set_path_override(path, wv if path != 1 else 0, c)
            compare_mx(run_gpu_mx(pd_, rd, gd, w.eps, "bf16"), ref, "geometry %s" % ((path, wv, c),))
    finally:
        arf.arf_set_path_override(0)



@pytest.mark.parametrize("shape", [(2, 2048, 8192, "bf16", 8), (6, 2048, 7168, "f32", 4),
                                   (16, 2048, 4096, "bf16", 8), (3, 768, 8192, "f16", 8)])
def test_mxfp4_on_held_rows_every_row(shape):
    # shapes where the plan takes held rows for a call with an MXFP4 copy; every row against
    # the oracle
    n, t, h, pd, waves = shape
    ad = "f16" if pd == "f16" else "bf16"
    w = _case(n, t, h, pd, ad, 621, std=3.0)
    plan = arf.arf_get_plan_quant(n, t, h, {"bf16": 0, "f16": 1, "f32": 2}[pd],
                                  arf.ARF_QUANT_MXFP4)
    assert plan["path"] == 3 and plan["waves"] == waves, plan
    say("mxfp4 on held rows %s" % (shape,))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, pd, ad, quant="mxfp4")
    compare_mx(run_gpu_mx(pd_, rd, gd, w.eps, ad), ref, "mxfp4 held %s" % (shape,))

def test_mxfp4_zero_rows_and_full_size():
    say("mxfp4 zero rows")
    h = 2048
    z = torch.zeros((2, 3, h), dtype=torch.bfloat16, device=DEV)
    got = run_gpu_mx(z, z[0].clone(), torch.ones(h, dtype=torch.bfloat16, device=DEV), 1e-6, "bf16")
    assert np.all(got["scales"] == 0) and np.all((got["codes"] & 7) == 0)
    say("mxfp4 c4 size, every row")
    w = workloads.WORKLOADS["c4"]
    p, r, g = workloads.generate(w, DEV)
    t = w.tokens
    got = run_gpu_mx(p, r, g, w.eps, "bf16")
    for b in range(0, t, 2048):
        e = min(t, b + 2048)
        say("mxfp4 c4 rows %d..%d" % (b, e))
        ref = run_oracle(p[:, b:e].contiguous(), r[b:e].contiguous(), g, w.eps, "bf16", "bf16",
                         quant="mxfp4")
        compare_mx({k: v[b:e] for k, v in got.items()}, ref, "c4 rows %d..%d" % (b, e))
    del p, r


# ---- size extremes ---------------------------------------------------------------------------

def test_many_tokens_small_rows():
    # 300000 rows of 64: a grid of hundreds of thousands of workgroups (or wavefront rows)
    w = _case(2, 300000, 64, "bf16", "bf16", 1000, quant="per_token")
    say("many tokens t=300000 h=64")
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    compare(run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_token"), ref, "t=300000")
    try:   # the same through one row per wavefront
        arf.arf_set_path_override(1)
        compare(run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_token"), ref, "t=300000 per wave")
    finally:
        arf.arf_set_path_override(0)


def test_launch_beyond_2pow32_work_items():
    # 2^26 + 5 rows of 8 elements on one row per wavefront: 2^32 + 1280 work-items, more than
    # one dispatch holds; the call runs as two kernels split at a row boundary. Rows around
    # the split, and the first and last rows, against the oracle.
    n, t, h = 1, (1 << 26) + 5, 8
    w = _case(n, t, h, "bf16", "bf16", 1300)
    say("launch beyond 2^32 work-items: t=%d h=%d" % (t, h))
    plan = arf.arf_get_plan(n, t, h, 0)
    assert plan["path"] == 1
    split = ((2 ** 32 - 1) // 256) * 4
    assert split < t
    p, r, g = workloads.generate(w, DEV)
    rout = torch.full((t, h), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    nout = torch.full((t, h), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    arf.arf_reduce_add_rmsnorm(p, r, g, w.eps, residual_out=rout, norm_out=nout)
    torch.cuda.synchronize()
    for b, e in ((0, 1024), (split - 1024, split + 5), (t - 1024, t)):
        say("rows %d..%d" % (b, e))
        ref = run_oracle(p[:, b:e].contiguous().cpu(), r[b:e].cpu(), g.cpu(), w.eps, "bf16", "bf16")
        got = {"residual_out": workloads.to_bits(rout[b:e]), "norm_out": workloads.to_bits(nout[b:e])}
        compare(got, ref, "rows %d..%d" % (b, e))
    del p, r, rout, nout


def test_partials_above_4_gib():
    # 16 shards x 16384 x 16384 bf16 = 8 GiB of partials: 64-bit offsets beyond 2^32 bytes
    w = workloads.Workload("huge", 16, 16384, 16384, "bf16", "bf16", 1.0, 1.0, 1e-6,
                           "per_token", 77)
    say("partials of 8 GiB (n=16 t=16384 h=16384)")
    p, r, g = workloads.generate(w, DEV)
    t, h = w.tokens, w.hidden
    rout = torch.empty((t, h), dtype=torch.bfloat16, device=DEV)
    nout = torch.empty((t, h), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((t, h), dtype=torch.uint8, device=DEV)
    sc = torch.empty((t,), dtype=torch.float32, device=DEV)
    arf.arf_reduce_add_rmsnorm_quant(p, r, g, w.eps, q, arf.ARF_QUANT_PER_TOKEN, scale_out=sc,
                                     residual_out=rout, norm_out=nout)
    torch.cuda.synchronize()
    rows = [0, 1, 8191, 8192, 12345, t - 1]
    idx = torch.tensor(rows, device=DEV)
    ref = run_oracle(p[:, idx].contiguous(), r[idx].contiguous(), g, w.eps, "bf16", "bf16",
                     quant="per_token")
    got = {"residual_out": workloads.to_bits(rout[idx]), "norm_out": workloads.to_bits(nout[idx]),
           "quant_out": q[idx].cpu().numpy(), "scale_out": sc[idx].cpu().numpy()}
    compare(got, ref, "8 GiB partials")
    del p, r, rout, nout, q
    torch.cuda.empty_cache()


# ---- rows claimed from a counter ----------------------------------------------------------

def test_claimed_rows_on_more_streams_than_counters():
    # 264 streams, more than the 256 counters of a device: each stream runs every-row-
    # claimed calls of two sizes one after another; the streams that find no free counter
    # take rows by workgroup index. Every output must equal the oracle's.
    w = _case(4, 70, 1024, "bf16", "bf16", 611, quant="per_token")
    w2 = _case(4, 33, 1024, "bf16", "bf16", 611, quant="per_token")
    say("claimed rows on 264 streams")
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    ref2 = run_oracle(p[:, :33].contiguous(), r[:33].contiguous(), g, w.eps, "bf16", "bf16",
                      quant="per_token")
    t, h = w.tokens, w.hidden
    pd33, rd33 = pd_[:, :33].contiguous(), rd[:33].contiguous()   # alive until the end
    streams = [torch.cuda.Stream() for _ in range(264)]
    outs = []
    torch.cuda.synchronize()
    try:
        arf.arf_set_path_override(4)
        for k, st in enumerate(streams):
            o = {"residual_out": Out((t, h), torch.bfloat16), "norm_out": Out((t, h), torch.bfloat16),
                 "quant_out": Out((t, h), torch.uint8), "scale_out": Out((t,), torch.float32)}
            o2 = {"residual_out": Out((33, h), torch.bfloat16), "norm_out": Out((33, h), torch.bfloat16),
                  "quant_out": Out((33, h), torch.uint8), "scale_out": Out((33,), torch.float32)}
            torch.cuda.synchronize()
            for oo, pp, rr in ((o, pd_, rd), (o2, pd33, rd33), (o, pd_, rd)):
                arf.arf_reduce_add_rmsnorm_quant(
                    pp, rr, gd, w.eps, oo["quant_out"].t, arf.ARF_QUANT_PER_TOKEN,
                    scale_out=oo["scale_out"].t, residual_out=oo["residual_out"].t,
                    norm_out=oo["norm_out"].t, stream=st)
            outs.append((o, o2))
        torch.cuda.synchronize()
    finally:
        arf.arf_set_path_override(0)
    for k, (o, o2) in enumerate(outs):
        for oo, rf, label in ((o, ref, "stream %d" % k), (o2, ref2, "stream %d (33 rows)" % k)):
            got = {}
            for name, x in oo.items():
                assert x.canary_ok(), (label, name)
                got[name] = x.t.cpu().numpy() if name in ("quant_out", "scale_out") else workloads.to_bits(x.t)
            compare(got, rf, label)


def test_claimed_rows_on_recreated_streams():
    # HIP gives a new stream the handle of one just destroyed, and with it that handle's
    # counter. Six streams are created through the HIP runtime in turn; each runs two
    # every-row-claimed calls and is destroyed right after them, with the last call
    # possibly still pending. Every output must equal the oracle's.
    hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch has loaded (same soname)
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    w = _case(4, 70, 1024, "bf16", "bf16", 613, quant="per_token")
    say("claimed rows on 6 streams created and destroyed in turn")
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    t, h = w.tokens, w.hidden
    outs, handles = [], []
    for k in range(6):
        o = {"residual_out": Out((t, h), torch.bfloat16), "norm_out": Out((t, h), torch.bfloat16),
             "quant_out": Out((t, h), torch.uint8), "scale_out": Out((t,), torch.float32)}
        torch.cuda.synchronize()   # the outputs' poison is written before the raw stream runs
        s = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(s)) == 0
        handles.append(s.value)
        try:
            arf.arf_set_path_override(4)
            for _ in range(2):
                arf.arf_reduce_add_rmsnorm_quant(
                    pd_, rd, gd, w.eps, o["quant_out"].t, arf.ARF_QUANT_PER_TOKEN,
                    scale_out=o["scale_out"].t, residual_out=o["residual_out"].t,
                    norm_out=o["norm_out"].t, stream=s.value)
        finally:
            arf.arf_set_path_override(0)
            assert hip.hipStreamDestroy(s) == 0
        outs.append(o)
    torch.cuda.synchronize()
    say("stream handles: %d distinct of 6" % len(set(handles)))
    for k, o in enumerate(outs):
        got = {}
        for name, x in o.items():
            assert x.canary_ok(), (k, name)
            got[name] = x.t.cpu().numpy() if name in ("quant_out", "scale_out") else workloads.to_bits(x.t)
        compare(got, ref, "recreated stream %d" % k)


def test_claim_plan_fp32_partials_every_row():
    # a shape the plan sends to claimed rows (4 fp32 shards of 4096 x 7168: 16 rows per
    # compute unit, 154 KiB per row), every row against the oracle
    w = _case(4, 4096, 7168, "f32", "bf16", 612)
    plan = arf.arf_get_plan(4, 4096, 7168, 2)
    assert plan["path"] == 4, plan
    say("claim plan %s" % plan)
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "f32", "bf16")
    got = run_gpu(pd_, rd, gd, w.eps, "bf16")
    compare(got, ref, "4 x 4096 x 7168 f32, claimed rows")


@pytest.mark.parametrize("shape", [(8, 8192, 2048, "bf16", "per_token"),
                                   (4, 8192, 8192, "bf16", None)])
def test_split_claim_plans_every_row(shape):
    # shapes the plan sends to claims spread over several counters: 44 KiB rows (4
    # counters, 4 workgroups per CU, the first 1024 workgroups keep their row) and 112 KiB
    # rows (2 counters, 2 per CU); every row against the oracle, twice on one stream (the
    # second call finds the counters the first left at 0)
    n, t, h, pd, quant = shape
    w = _case(n, t, h, pd, "bf16", 614, quant=quant)
    plan = arf.arf_get_plan(n, t, h, 0)
    assert plan["path"] == 4 and plan["grid"] == t + 512, plan
    say("split claims %s" % (shape,))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, pd, "bf16", quant=quant)
    for k in range(2):
        got = run_gpu(pd_, rd, gd, w.eps, "bf16", quant=quant)
        compare(got, ref, "%s, call %d" % (shape, k))


HIP_STREAM_PER_THREAD = 2   # the value of hipStreamPerThread in hip_runtime_api.h


def test_per_thread_and_legacy_default_streams():
    # a shape whose plan claims rows, on the per-thread default stream (where the library
    # takes rows by workgroup index instead: one handle stands for a different stream in
    # every thread) and on the legacy default stream (handle 0, which claims); every row
    # against the oracle
    n, t, h = 8, 8192, 2048
    w = _case(n, t, h, "bf16", "bf16", 618, quant="per_token")
    assert arf.arf_get_plan(n, t, h, 0)["path"] == 4
    say("per-thread and legacy default streams")
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    for handle in (HIP_STREAM_PER_THREAD, 0):
        got = run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_token", stream=handle)
        compare(got, ref, "stream handle %d" % handle)


@pytest.mark.parametrize("shape", [(2, 2048, 7168, "bf16"), (4, 4096, 4096, "f16"),
                                   (3, 1536, 8192, "bf16"), (8, 2048, 7168, "bf16"),
                                   (16, 1536, 4096, "f16")])
def test_held_rows_with_eight_wavefronts_every_row(shape):
    # 16-bit partials in the held-row region (any shard count): the plan takes the held
    # kernel with 8 wavefronts (half the chunks per lane); every row against the oracle,
    # then the same call with 4 wavefronts forced (the general form beyond 4 shards), which
    # must give the same outputs within the tolerance
    n, t, h, dt = shape
    w = _case(n, t, h, dt, dt, 615, quant=None)
    plan = arf.arf_get_plan(n, t, h, {"bf16": 0, "f16": 1}[dt])
    assert plan["path"] == 3 and plan["waves"] == 8, plan
    say("held rows, 8 wavefronts, %s" % (shape,))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, dt, dt)
    compare(run_gpu(pd_, rd, gd, w.eps, dt), ref, "%s, 8 wavefronts" % (shape,))
    try:
        arf.arf_set_path_override(3, 4, 0)
        assert arf.arf_get_plan(n, t, h, {"bf16": 0, "f16": 1}[dt])["waves"] == 4
        got4 = run_gpu(pd_, rd, gd, w.eps, dt)
    finally:
        arf.arf_set_path_override(0)
    compare(got4, ref, "%s, 4 wavefronts" % (shape,))


@pytest.mark.parametrize("shape", [(8, 2048, 7168), (16, 1536, 4096)])
def test_held_rows_fp32_many_shards_every_row(shape):
    # fp32 partials beyond 4 shards in the held-row region: the plan takes the 4-wavefront
    # form without a quantised copy; every row against the oracle
    n, t, h = shape
    w = _case(n, t, h, "f32", "bf16", 616, quant=None)
    plan = arf.arf_get_plan(n, t, h, 2)
    assert plan["path"] == 3 and plan["waves"] == 4, plan
    say("held rows, fp32 partials, %s" % (shape,))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, "f32", "bf16")
    compare(run_gpu(pd_, rd, gd, w.eps, "bf16"), ref, "f32 %s, held rows" % (shape,))



@pytest.mark.parametrize("pd,quant", [("bf16", None), ("bf16", "per_token"), ("f32", "per_tensor")])
def test_held_rows_beyond_64_per_batch(pd, quant):
    # The held-row kernel forms the inverse RMS of its first 64 held rows in parallel, one
    # per lane, and of any further row in turn. Rows of 64 elements take about 700 to a
    # batch, so 25677 rows give each of the 256 workgroups one batch of 100 or 101 rows
    # (4 shards; 8 wavefronts without a copy, 4 with one); every row against the oracle.
    n, t, h = 4, 25677, 64
    w = _case(n, t, h, pd, "bf16", 617, quant=quant)
    say("held rows beyond 64 per batch, %s %s" % (pd, quant))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, pd, "bf16", quant=quant,
                     scale_in=0.02 if quant == "per_tensor" else None)
    try:
        arf.arf_set_path_override(3)
        plan = arf.arf_get_plan(n, t, h, {"bf16": 0, "f32": 2}[pd])
        assert plan["path"] == 3 and plan["grid"] == min(t, torch.cuda.get_device_properties(0).multi_processor_count), plan
        got = run_gpu(pd_, rd, gd, w.eps, "bf16", quant=quant, scale=0.02)
    finally:
        arf.arf_set_path_override(0)
    compare(got, ref, "held rows, %s %s, %d rows of %d" % (pd, quant, t, h))



@pytest.mark.parametrize("shape", [(4, 2048, 7168, "bf16", 4), (2, 1024, 8192, "f16", 8),
                                   (8, 1536, 7168, "f32", 4), (3, 1536, 6144, "bf16", 4),
                                   (8, 2048, 7168, "bf16", 8), (3, 768, 4096, "f16", 8),
                                   (12, 2048, 4096, "bf16", 8), (6, 2048, 4096, "f32", 4),
                                   (2, 768, 7168, "f32", 4)])
def test_held_rows_with_a_per_tensor_copy_every_row(shape):
    # shapes where the plan takes held rows for a call with a per-tensor fp8 copy (the
    # general form, 4 or 8 wavefronts); every row against the oracle
    n, t, h, pd, waves = shape
    ad = "f16" if pd == "f16" else "bf16"
    w = _case(n, t, h, pd, ad, 619, quant="per_tensor")
    plan = arf.arf_get_plan_quant(n, t, h, {"bf16": 0, "f16": 1, "f32": 2}[pd],
                                  arf.ARF_QUANT_PER_TENSOR)
    assert plan["path"] == 3 and plan["waves"] == waves, plan
    say("held rows, per-tensor copy, %s" % (shape,))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, pd, ad, quant="per_tensor", scale_in=0.03)
    compare(run_gpu(pd_, rd, gd, w.eps, ad, quant="per_tensor", scale=0.03), ref,
            "per-tensor %s, held rows" % (shape,))


@pytest.mark.parametrize("shape", [(8, 2048, 7168, "bf16", 8), (4, 2048, 8192, "f16", 8),
                                   (16, 3072, 4096, "bf16", 8), (4, 2048, 7168, "bf16", 4)])
def test_held_rows_forced_with_per_token_scales_every_row(shape):
    # held rows forced on calls with a per-token copy: batches of several rows per
    # workgroup, whose maxima are formed before any code is written; every row against
    # the oracle
    n, t, h, pd, waves = shape
    ad = "f16" if pd == "f16" else "bf16"
    w = _case(n, t, h, pd, ad, 620, quant="per_token")
    say("held rows forced, per-token scales, %s" % (shape,))
    (p, r, g), (pd_, rd, gd) = upload(w)
    ref = run_oracle(p, r, g, w.eps, pd, ad, quant="per_token")
    try:
        arf.arf_set_path_override(3, waves, 0)
        got = run_gpu(pd_, rd, gd, w.eps, ad, quant="per_token")
    finally:
        arf.arf_set_path_override(0)
    compare(got, ref, "held rows forced, per-token, %s" % (shape,))

# ---- HIP graph capture --------------------------------------------------------------------

@pytest.mark.parametrize("path", [0, 4])
def test_graph_capture_and_replay(path):
    # the fused call captured into a graph on a side stream, replayed with eager work
    # (poisoning the outputs) in between; every replay must equal the eager result. With
    # path 4 the eager call claims its rows and the captured one takes them by workgroup
    # index (a graph may be replayed on any stream): the same bits
    w = workloads.WORKLOADS["c1"]
    say("graph capture / replay %s path %d" % (w.name, path))
    arf.arf_set_path_override(path)
    try:
        _graph_capture_and_replay(w)
    finally:
        arf.arf_set_path_override(0)


def _graph_capture_and_replay(w):
    (p, r, g), (pd_, rd, gd) = upload(w)
    t, h = w.tokens, w.hidden
    eager = run_gpu(pd_, rd, gd, w.eps, "bf16", quant="per_token")
    rout = torch.empty((t, h), dtype=torch.bfloat16, device=DEV)
    nout = torch.empty((t, h), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((t, h), dtype=torch.uint8, device=DEV)
    sc = torch.empty((t,), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up launch outside the capture
        arf.arf_reduce_add_rmsnorm_quant(pd_, rd, gd, w.eps, q, arf.ARF_QUANT_PER_TOKEN,
                                         scale_out=sc, residual_out=rout, norm_out=nout)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        arf.arf_reduce_add_rmsnorm_quant(pd_, rd, gd, w.eps, q, arf.ARF_QUANT_PER_TOKEN,
                                         scale_out=sc, residual_out=rout, norm_out=nout)
    for k in range(4):
        for o in (rout, nout):
            o.view(torch.int16).fill_(-1)
        q.fill_(0xFF)
        sc.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"residual_out": workloads.to_bits(rout), "norm_out": workloads.to_bits(nout),
               "quant_out": q.cpu().numpy(), "scale_out": sc.cpu().numpy()}
        for key in eager:
            assert np.array_equal(got[key], eager[key]), (k, key)


def test_graph_capture_of_mixed_calls():
    # several different calls in one captured graph: MXFP4 over a row range with
    # partial-type accumulation, per-tensor fp8, and the token-slice composition (reduce a
    # slice, then the epilogue over all rows from the reduced values); every replay,
    # with the outputs poisoned eagerly in between, equals the same calls run eagerly
    w = workloads.WORKLOADS["c2"]
    say("graph capture of mixed calls %s" % w.name)
    (p, r, g), (pd_, rd, gd) = upload(w)
    t, h = w.tokens, w.hidden
    bf = torch.bfloat16
    scale = torch.tensor([0.02], dtype=torch.float32, device=DEV)

    def outputs():
        return dict(r1=torch.empty((t, h), dtype=bf, device=DEV),
                    n1=torch.empty((t, h), dtype=bf, device=DEV),
                    q1=torch.empty((t, h // 2), dtype=torch.uint8, device=DEV),
                    s1=torch.empty((t, h // 32), dtype=torch.uint8, device=DEV),
                    n2=torch.empty((t, h), dtype=bf, device=DEV),
                    q2=torch.empty((t, h), dtype=torch.uint8, device=DEV),
                    sums=torch.empty((t, h), dtype=bf, device=DEV),
                    r3=torch.empty((t, h), dtype=bf, device=DEV),
                    n3=torch.empty((t, h), dtype=bf, device=DEV))

    def poison(o):
        for v in o.values():
            v.view(torch.uint8).fill_(0xFF)

    def calls(o, stream=None):
        arf.arf_fused_epilogue(pd_, rd, gd, w.eps, residual_out=o["r1"], norm_out=o["n1"],
                               quant_out=o["q1"], mode=arf.ARF_QUANT_MXFP4, scale_out=o["s1"],
                               accumulate=arf.ARF_ACC_PARTIAL, row_begin=0, row_count=40,
                               stream=stream)
        arf.arf_reduce_add_rmsnorm_quant(pd_, rd, gd, w.eps, o["q2"], arf.ARF_QUANT_PER_TENSOR,
                                         scale_in=scale, norm_out=o["n2"], stream=stream)
        arf.arf_reduce_rows(pd_, o["sums"], row_begin=0, row_count=t, stream=stream)
        arf.arf_reduce_add_rmsnorm(o["sums"].view(1, t, h), rd, gd, w.eps, residual_out=o["r3"],
                                   norm_out=o["n3"], stream=stream)

    ref = outputs()
    poison(ref)
    calls(ref)
    torch.cuda.synchronize()
    ref = {k: v.view(torch.uint8).cpu().numpy() for k, v in ref.items()}
    # the token-slice composition gives the oneshot result (same rounding steps)
    assert np.array_equal(ref["n3"], ref["n2"])
    assert np.all(ref["r1"].reshape(t, -1)[40:] == 0xFF)   # rows outside the range
    o = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        calls(o, stream=side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        calls(o)
    for k in range(4):
        poison(o)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key, v in o.items():
            assert np.array_equal(v.view(torch.uint8).cpu().numpy(), ref[key]), (k, key)

def test_stream_mix_writes_exactly_its_range():
    for rb, wb, units in ((1 << 20, 1 << 18, 0), (3 * 16384 + 48, 0, 0), (0, 5 * 16384 + 16, 3),
                          (64 << 20, 16 << 20, 1024)):
        say("stream mix read %d write %d units %d" % (rb, wb, units))
        src = torch.randint(0, 256, (max(rb, 16),), dtype=torch.uint8, device=DEV)
        dst = torch.full((wb + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        arf.arf_stream_mix(dst, wb, src, rb, units)
        torch.cuda.synchronize()
        assert bool((dst[wb:] == CANARY).all())
        if wb:   # every 16-byte word of the range was written (none keeps the canary)
            words = dst[:wb].view(-1, 16)
            assert not bool((words == CANARY).all(dim=1).any())


# ---- special values ---------------------------------------------------------------------------

def _same_or_both_nan16(a, b, act):
    fa, fb = oracle.act_to_f32(a, act), oracle.act_to_f32(b, act)
    both_nan = np.isnan(fa) & np.isnan(fb)
    return bool(np.all(both_nan | (a == b)))


@pytest.mark.parametrize("value", ["nan", "inf", "-inf", "negzero"])
def test_special_values_mxfp4(value):
    # the MXFP4 copy of rows holding NaN, +-inf or -0: block scales and every code equal to
    # the oracle's (NaN and infinities saturate to +-6, NaN stays out of the block maximum)
    say("special value %s, mxfp4" % value)
    w = _case(4, 6, 1024, "bf16", "bf16", 1150)
    p, r, g = workloads.generate(w, "cpu")
    p = p.clone()
    if value == "negzero":
        p.fill_(-0.0)
        r = torch.full_like(r, -0.0)
    else:
        p[2, 3, 17] = float(value)
        p[0, 5, 1000] = float(value)
    from helpers import unpack_fp4
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="mxfp4")
    got = run_gpu_mx(p.to(DEV), r.to(DEV), g.to(DEV), w.eps, "bf16")
    assert _same_or_both_nan16(got["residual_out"], ref["residual_out"], "bf16")
    assert _same_or_both_nan16(got["norm_out"], ref["norm_out"], "bf16")
    assert np.array_equal(got["scales"], ref["scale_out"])
    assert np.array_equal(got["codes"], unpack_fp4(ref["quant_out"]))


@pytest.mark.parametrize("value", ["nan", "inf", "-inf", "negzero"])
def test_special_values_match_the_oracle(value):
    say("special value %s" % value)
    w = _case(4, 6, 1024, "bf16", "bf16", 1100, quant="per_token")
    p, r, g = workloads.generate(w, "cpu")
    p = p.clone()
    if value == "negzero":
        p.fill_(-0.0)
        r = torch.full_like(r, -0.0)
    else:
        p[2, 3, 17] = float(value)
        p[0, 5, 1000] = float(value)
    ref = run_oracle(p, r, g, w.eps, "bf16", "bf16", quant="per_token")
    got = run_gpu(p.to(DEV), r.to(DEV), g.to(DEV), w.eps, "bf16", quant="per_token")
    assert _same_or_both_nan16(got["residual_out"], ref["residual_out"], "bf16")
    assert _same_or_both_nan16(got["norm_out"], ref["norm_out"], "bf16")
    qg, qr = got["quant_out"], ref["quant_out"]
    nan_codes = (qr & 0x7F) == 0x7F
    assert np.array_equal((qg & 0x7F) == 0x7F, nan_codes)
    assert np.array_equal(qg[~nan_codes], qr[~nan_codes])
    sg, sr = got["scale_out"], ref["scale_out"]
    assert np.array_equal(np.isnan(sg), np.isnan(sr)) and np.array_equal(sg[~np.isnan(sr)], sr[~np.isnan(sr)])


# ---- seeded random general calls -------------------------------------------------------------

def _random_case(rng, k):
    """One general call: sizes, types, accumulation, row range, output subset, in place,
    quantised copy and eps, drawn from a fixed-seed generator."""
    pd, ad = [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16"), ("f32", "f16")][rng.integers(4)]
    n = int(rng.integers(1, 17))
    t = int(rng.choice([0, 1, 2, 3, 5, 17, 64, 130, 300]))
    h = 8 * int(np.exp(rng.uniform(0.0, np.log(2500.0))))
    quant = [None, "per_tensor", "per_token", "mxfp4"][rng.integers(4)]
    if quant == "mxfp4":
        h = -(-h // 32) * 32
    while n * t * h > (1 << 22):   # bound the case's size
        t //= 2
    res, norm = bool(rng.random() < 0.8), bool(rng.random() < 0.8)
    if quant is None and not (res or norm):
        norm = True
    begin = int(rng.integers(0, t + 1))
    count = int(rng.integers(-1, t - begin + 1))
    return dict(n=n, t=t, h=h, pd=pd, ad=ad, quant=quant, res=res, norm=norm,
                in_place=res and bool(rng.random() < 0.3), begin=begin, count=count,
                acc=["f32", "partial"][rng.integers(2)],
                eps=float(rng.choice([0.0, 1e-6, 1e-5, 0.1])),
                scale=float(rng.uniform(1e-3, 0.1)), seed=9000 + k)


@pytest.mark.parametrize("path", [0, 3, 4])
def test_seeded_random_general_calls_match_the_oracle(path):
    # path 0: the plan; path 3: the held-row kernel forced on every call (one or several
    # batches per workgroup, row ranges, in place, every quantised copy); path 4: every row
    # of every call claimed from the stream's counter
    try:
        arf.arf_set_path_override(path)
        _random_general_calls(path)
    finally:
        arf.arf_set_path_override(0)


def _random_general_calls(path):
    rng = np.random.default_rng(20261202)
    for k in range(200):
        c = _random_case(rng, k)
        if path == 3 and c["h"] > 16384:
            continue    # the held-row kernel covers rows of up to 16384 elements
        w = _case(c["n"], c["t"], c["h"], c["pd"], c["ad"], c["seed"], eps=c["eps"])
        say("random call %d: %s" % (k, c))
        (p, r, g), (pd_, rd, gd) = upload(w)
        t, h, adt = c["t"], c["h"], TORCH[c["ad"]]
        rows = slice(c["begin"], t if c["count"] < 0 else c["begin"] + c["count"])
        # GPU: every output poisoned and guarded; in place writes the residual over a copy
        rin = rd.clone() if c["in_place"] else rd
        rout = None if (not c["res"] or c["in_place"]) else Out((t, h), adt)
        nout = Out((t, h), adt) if c["norm"] else None
        q = sout = None
        sin = None
        kw = {}
        if c["quant"] == "mxfp4":
            q, sout = Out((t, h // 2), torch.uint8), Out((t, h // 32), torch.uint8)
            kw = dict(quant_out=q.t, mode=arf.ARF_QUANT_MXFP4, scale_out=sout.t)
        elif c["quant"] == "per_token":
            q, sout = Out((t, h), torch.uint8), Out((t,), torch.float32)
            kw = dict(quant_out=q.t, mode=arf.ARF_QUANT_PER_TOKEN, scale_out=sout.t)
        elif c["quant"] == "per_tensor":
            q = Out((t, h), torch.uint8)
            sin = torch.tensor([c["scale"]], dtype=torch.float32, device=DEV)
            kw = dict(quant_out=q.t, mode=arf.ARF_QUANT_PER_TENSOR, scale_in=sin)
        arf.arf_fused_epilogue(pd_, rin, gd, w.eps,
                               residual_out=rin if c["in_place"] else (rout.t if rout else None),
                               norm_out=nout.t if nout else None, row_begin=c["begin"],
                               row_count=c["count"],
                               accumulate=arf.ARF_ACC_PARTIAL if c["acc"] == "partial" else arf.ARF_ACC_F32,
                               **kw)
        torch.cuda.synchronize()
        # oracle: the same call, unwritten rows left at the poison byte
        rb = workloads.to_bits(r)
        ref = oracle.reduce_add_rmsnorm(
            workloads.to_bits(p), rb.copy() if c["in_place"] else rb, workloads.to_bits(g),
            w.eps, partial_dtype=c["pd"], act_dtype=c["ad"],
            residual_out=c["res"], norm_out=c["norm"], quant=c["quant"],
            scale_in=c["scale"] if c["quant"] == "per_tensor" else None,
            residual_out_array=None, accumulate=c["acc"], rows=(c["begin"], c["count"]),
            out_init=POISON, n_threads=THREADS)
        if c["in_place"]:
            exp = rb.copy()
            exp[rows] = oracle.reduce_add_rmsnorm(
                workloads.to_bits(p), rb, workloads.to_bits(g), w.eps, partial_dtype=c["pd"],
                act_dtype=c["ad"], norm_out=False, accumulate=c["acc"],
                rows=(c["begin"], c["count"]), n_threads=THREADS)["residual_out"][rows]
            assert np.array_equal(workloads.to_bits(rin), exp), k
        got = {}
        for name, o in (("residual_out", rout), ("norm_out", nout), ("quant_out", q),
                        ("scale_out", sout)):
            if o is None:
                continue
            assert o.canary_ok(), (k, name)
            got[name] = workloads.to_bits(o.t) if o.t.dtype in (torch.bfloat16, torch.float16) \
                else o.t.cpu().numpy()
            if t:
                outside = np.ones(t, bool)
                outside[rows] = False
                raw = o.raw[:o.nbytes].cpu().numpy().reshape(t, -1)
                assert np.all(raw[outside] == POISON), (k, name, "a row outside the range was written")
        if rows.stop <= rows.start:
            continue
        ins = {kk: v[rows] for kk, v in got.items()}
        refs = {kk: v[rows] for kk, v in ref.items() if kk in got}
        if c["quant"] == "mxfp4":
            from helpers import unpack_fp4
            compare({kk: ins[kk] for kk in ins if kk in ("residual_out", "norm_out")},
                    {kk: refs[kk] for kk in refs if kk in ("residual_out", "norm_out")},
                    "case %d" % k, min_exact=0.0)
            assert np.array_equal(ins["scale_out"], refs["scale_out"]), k
            d = np.abs(_ord4(unpack_fp4(ins["quant_out"])) - _ord4(unpack_fp4(refs["quant_out"])))
            assert d.size == 0 or d.max() <= 1, k
        else:
            compare(ins, refs, "case %d" % k, min_exact=0.0)
