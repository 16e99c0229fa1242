"""CPU checks of the C ABI: the library loads, exports every symbol include/arfuse.h
declares, and rejects bad arguments before any device call. No kernel is launched:
every call below fails validation or is empty (tokens == 0), except the no-device case,
which only runs where no GPU is present."""
import ctypes
import os
import re

import pytest

import shard_reduce_residual_amd as arf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arfuse.h")

# fake, well-aligned, non-overlapping device addresses: never dereferenced, because
# every call using them fails validation first
P, R, RO, G, NO, Q, S = (0x10000000 * k for k in range(1, 8))


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(arf_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = arf.lib()
    names = declared_symbols()
    assert len(names) == 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(arf.SIGNATURES)


def test_library_exports_nothing_else():
    # the dynamic symbol table holds the C ABI only (the build's version script keeps the
    # kernels' launchers and host stubs local)
    import shutil
    import subprocess
    if not shutil.which("nm"):
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", arf.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    names = sorted(line.split()[-1] for line in out.splitlines() if line.strip())
    assert names == declared_symbols(), names[:20]


def test_version_and_status_strings():
    assert arf.arf_version() == 400
    for code, name in enumerate(arf.STATUS):
        assert arf.arf_status_string(code).startswith(name)
    assert "unknown" in arf.arf_status_string(99)


def call(**kw):
    a = dict(partials=P, n=2, tokens=4, hidden=64, pdt=0, adt=0, rin=R, rout=RO, gamma=G,
             eps=1e-6, nout=NO)
    a.update(kw)
    return arf.lib().arf_reduce_add_rmsnorm(a["partials"], a["n"], a["tokens"], a["hidden"],
                                            a["pdt"], a["adt"], a["rin"], a["rout"],
                                            a["gamma"], a["eps"], a["nout"], None)


def callq(**kw):
    a = dict(partials=P, n=2, tokens=4, hidden=64, pdt=0, adt=0, rin=R, rout=RO, gamma=G,
             eps=1e-6, nout=NO, q=Q, mode=1, sin=None, sout=S)
    a.update(kw)
    return arf.lib().arf_reduce_add_rmsnorm_quant(
        a["partials"], a["n"], a["tokens"], a["hidden"], a["pdt"], a["adt"], a["rin"],
        a["rout"], a["gamma"], a["eps"], a["nout"], a["q"], a["mode"], a["sin"], a["sout"],
        None)


OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, NOOUT, VALUE, HIP = range(9)


@pytest.mark.parametrize("kw,want", [
    (dict(partials=None), NULL), (dict(rin=None), NULL), (dict(gamma=None), NULL),
    (dict(rout=None, nout=None), NOOUT),
    (dict(n=0), SHAPE), (dict(n=17), SHAPE), (dict(tokens=-1), SHAPE),
    (dict(tokens=2 ** 31), SHAPE), (dict(hidden=0), SHAPE), (dict(hidden=12), SHAPE),
    (dict(hidden=65544), SHAPE),
    (dict(adt=2), DTYPE), (dict(adt=3), DTYPE), (dict(pdt=1, adt=0), DTYPE),
    (dict(pdt=0, adt=1), DTYPE),
    (dict(eps=-1e-6), VALUE), (dict(eps=float("inf")), VALUE), (dict(eps=float("nan")), VALUE),
    (dict(partials=P + 8), ALIGN), (dict(rout=RO + 2), ALIGN), (dict(gamma=G + 4), ALIGN),
    (dict(nout=R), ALIAS), (dict(rout=P), ALIAS), (dict(nout=RO), ALIAS),
    (dict(rout=R + 16), ALIAS), (dict(nout=G), ALIAS),
    (dict(tokens=0), OK), (dict(tokens=0, rout=R), OK),
])
def test_validation(kw, want):
    assert call(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), NULL), (dict(mode=1, sout=None), NULL), (dict(mode=0, sin=None), NULL),
    (dict(mode=2), VALUE), (dict(mode=-1), VALUE),
    (dict(sout=S + 2), ALIGN), (dict(q=Q + 8), ALIGN),
    (dict(q=NO), ALIAS), (dict(sout=Q), ALIAS), (dict(mode=0, sin=RO, sout=None), ALIAS),
    (dict(rout=None, nout=None, tokens=0), OK),
    (dict(mode=0, sin=S, sout=None, tokens=0), OK),
])
def test_quant_validation(kw, want):
    assert callq(**kw) == want


def test_in_place_residual_passes_validation_and_empty_call_is_ok():
    # residual_out == residual_in is the one allowed overlap
    assert call(rout=R, tokens=0) == OK


def test_utility_entry_point_validation():
    L = arf.lib()
    assert L.arf_e4m3_encode(P, Q, 0, None) == OK
    assert L.arf_e4m3_encode(None, Q, 8, None) == NULL
    assert L.arf_e4m3_encode(P, Q, -1, None) == SHAPE
    assert L.arf_e4m3_encode(P + 2, Q, 8, None) == ALIGN
    assert L.arf_e4m3_encode(P, P + 4, 8, None) == ALIAS
    assert L.arf_e2m1_encode(P, Q, 0, None) == OK
    assert L.arf_e2m1_encode(None, Q, 8, None) == NULL
    assert L.arf_e2m1_encode(P, Q, -1, None) == SHAPE
    assert L.arf_e2m1_encode(P + 2, Q, 8, None) == ALIGN
    assert L.arf_e2m1_encode(P, P + 4, 8, None) == ALIAS
    assert L.arf_stream_copy(Q, P, 0, None) == OK
    assert L.arf_stream_copy(Q, P, 24, None) == SHAPE
    assert L.arf_stream_copy(Q, None, 32, None) == NULL
    assert L.arf_stream_copy(Q + 8, P, 32, None) == ALIGN
    assert L.arf_stream_copy(P + 16, P, 64, None) == ALIAS


def plan(n, t, h, pd=0, cus=256):
    return arf.arf_get_plan(n, t, h, pd, cus)


def test_plan_covers_the_row_and_follows_the_menu():
    try:
        for h in (8, 64, 264, 1024, 2048, 4096, 7168, 8192, 16384, 32768, 65536):
            for t in (1, 16, 128, 2048, 8192):
                for n in (2, 8):
                    p = plan(n, t, h)
                    lanes = 64 if p["path"] == 1 else 64 * p["waves"]
                    assert lanes * p["chunks"] * 8 >= h
                    assert p["chunks"] in (1, 2, 4, 8)
                    if p["path"] == 1:
                        assert p["waves"] == 4 and p["grid"] == (t + 3) // 4
                    elif p["path"] == 2:
                        assert p["waves"] in (4, 8, 16) and p["grid"] == t
                    elif p["path"] == 4:   # claimed rows: the rows plus the surplus,
                        # rounded up to a multiple of 8 * split (split 2 or 4)
                        assert p["waves"] == 4 and t >= 8 * 256
                        assert 0 <= p["grid"] - (t + max(64, t // 16)) < 32
                    else:   # held rows: one workgroup per CU, one batch of rows each;
                        # 8 wavefronts for 16-bit partials (these are bf16)
                        assert p["path"] == 3 and p["waves"] == 8
                        assert p["grid"] == min(t, 256) and t >= 3 * 256
                        assert -(-t // 256) * (2 * h + 96) <= 160 * 1024
    finally:
        arf.arf_set_path_override(0)


def test_plan_for_the_named_workloads():
    # geometries measured best on MI355X for these shapes
    assert plan(8, 8192, 16384) == {"path": 4, "waves": 4, "chunks": 8, "grid": 8192 + 512}
    assert plan(4, 2048, 7168, 2) == {"path": 3, "waves": 4, "chunks": 4, "grid": 256}
    assert plan(8, 128, 4096) == {"path": 2, "waves": 8, "chunks": 1, "grid": 128}
    assert plan(8, 64, 8192) == {"path": 2, "waves": 8, "chunks": 2, "grid": 64}
    assert plan(2, 16, 1024)["path"] == 2
    assert plan(4, 4096, 7168) == {"path": 2, "waves": 4, "chunks": 4, "grid": 4096}
    assert plan(4, 4096, 7168, 2) == {"path": 4, "waves": 4, "chunks": 4, "grid": 4096 + 256}
    assert plan(2, 1024, 4096) == {"path": 3, "waves": 8, "chunks": 1, "grid": 256}
    assert plan(8, 8192, 65536) == {"path": 2, "waves": 16, "chunks": 8, "grid": 8192}


def test_plan_few_rows():
    # fewer than 2 rows per CU: rows of <= 64 chunks one per wavefront, rows of <= 256
    # chunks 4 wavefronts per row (more would leave lanes idle), wider rows 8 wavefronts
    assert plan(2, 16, 1024) == {"path": 2, "waves": 4, "chunks": 1, "grid": 16}
    assert plan(8, 100, 2048) == {"path": 2, "waves": 4, "chunks": 1, "grid": 100}
    assert plan(8, 100, 2056) == {"path": 2, "waves": 8, "chunks": 1, "grid": 100}
    assert plan(8, 16, 512) == {"path": 1, "waves": 4, "chunks": 1, "grid": 4}
    assert plan(8, 1, 8) == {"path": 1, "waves": 4, "chunks": 1, "grid": 1}
    assert plan(8, 128, 4096)["waves"] == 8 and plan(8, 64, 8192)["waves"] == 8


def test_plan_row_per_wave_region():
    # one row per wavefront: rows of <= 128 chunks from 2 rows per CU, rows of <= 256
    # chunks from 8 rows per CU; never for wider rows
    assert plan(8, 511, 1024)["path"] == 2 and plan(8, 512, 1024)["path"] == 1
    assert plan(8, 8192, 1024) == {"path": 1, "waves": 4, "chunks": 2, "grid": 2048}
    assert plan(8, 2047, 2048)["path"] == 2 and plan(8, 2048, 2048)["path"] == 1
    assert plan(8, 8191, 2048) == {"path": 1, "waves": 4, "chunks": 4, "grid": 2048}
    assert plan(4, 16384, 2048)["path"] == 1            # 28 KiB per row: no claims
    assert plan(16, 16384, 1024)["path"] == 1           # 128 chunks: no claims
    assert plan(4, 8191, 2056, 2)["path"] == 2          # 257 chunks
    assert plan(4, 8192, 2056, 2)["path"] == 4          # 257 chunks, claimed from 32 per CU
    for t in (512, 1024, 2048, 4096, 8191):   # never one row per wavefront (held rows at
        assert plan(8, t, 4096)["path"] != 1      # 3-19 rows per CU)
    # the thresholds scale with the CU count
    assert plan(8, 1023, 2048, 0, 128)["path"] == 2 and plan(8, 1024, 2048, 0, 128)["path"] == 1


def test_plan_held_rows_region():
    # held rows only where measured faster: <= 4 shards, 4096 <= hidden <= 8192, 6 to 16
    # rows per CU, one batch per workgroup (LDS holds 11 rows of 7168, 9 of 8192)
    assert plan(4, 767, 7168, 2)["path"] != 3 and plan(4, 768, 7168, 2)["path"] == 3
    assert plan(4, 11 * 256, 7168, 2)["path"] == 3 and plan(4, 11 * 256 + 1, 7168, 2)["path"] == 2
    assert plan(2, 9 * 256, 8192)["path"] == 3 and plan(2, 9 * 256 + 1, 8192)["path"] == 2
    assert plan(4, 19 * 256, 4096)["path"] == 3 and plan(4, 19 * 256 + 1, 4096)["path"] != 3
    assert plan(5, 2048, 7168) == {"path": 3, "waves": 8, "chunks": 2, "grid": 256}
    assert plan(16, 4096, 4096)["path"] == 3
    # from 3 rows per CU, 16-bit (8 wavefronts) and fp32 (4) partials alike
    assert plan(8, 767, 4096)["path"] != 3 and plan(8, 768, 4096)["path"] == 3
    # fp32 partials: 4 wavefronts, beyond 4 shards where shards x chunks <= 48
    assert plan(5, 2048, 7168, 2) == {"path": 3, "waves": 4, "chunks": 4, "grid": 256}
    assert plan(12, 2048, 8192, 2)["path"] == 3 and plan(16, 2048, 4096, 2)["path"] == 3
    assert plan(16, 2048, 7168, 2)["path"] != 3
    assert plan(4, 2048, 4088)["path"] != 3 and plan(4, 2048, 4096)["path"] == 3
    assert plan(4, 2048, 8200)["path"] == 2
    # the thresholds scale with the CU count
    assert plan(4, 383, 7168, 2, 128)["path"] != 3 and plan(4, 384, 7168, 2, 128)["path"] == 3



def qplan(n, t, h, quant, pd=0, cus=256):
    return arf.arf_get_plan_quant(n, t, h, pd, quant, cus)


def test_plan_with_a_quantised_copy():
    # the plan of a call with a copy: ARF_QUANT_NONE is arf_get_plan's answer
    for args in [(4, 2048, 7168, 2), (8, 8192, 16384, 0), (2, 16, 1024, 0), (8, 64, 8192, 0)]:
        assert qplan(*args[:3], arf.ARF_QUANT_NONE, args[3]) == plan(*args)
    # held rows take no per-token copy
    assert qplan(4, 2048, 7168, arf.ARF_QUANT_PER_TOKEN, 2)["path"] == 2
    assert qplan(2, 2048, 8192, arf.ARF_QUANT_PER_TOKEN)["path"] != 3
    # an MXFP4 copy: the region without a copy, 9-16 16-bit shards from 8 rows per CU
    m = arf.ARF_QUANT_MXFP4
    assert qplan(4, 2048, 7168, m, 2) == plan(4, 2048, 7168, 2)
    assert qplan(2, 2048, 8192, m) == {"path": 3, "waves": 8, "chunks": 2, "grid": 256}
    assert qplan(8, 768, 4096, m)["path"] == 3 and qplan(8, 767, 4096, m)["path"] != 3
    assert qplan(16, 2047, 4096, m)["path"] != 3 and qplan(16, 2048, 4096, m)["path"] == 3
    assert qplan(1, 2048, 8192, m)["path"] == 3
    # a per-tensor copy. fp32 partials: 4 wavefronts, 2-8 shards, hidden 6144-8192 from 3
    # rows per CU, hidden 4096 from 8
    t = arf.ARF_QUANT_PER_TENSOR
    assert qplan(4, 2048, 7168, t, 2) == {"path": 3, "waves": 4, "chunks": 4, "grid": 256}
    assert qplan(8, 1536, 7168, t, 2)["path"] == 3 and qplan(9, 1536, 7168, t, 2)["path"] != 3
    assert qplan(4, 768, 8192, t, 2)["path"] == 3 and qplan(4, 767, 8192, t, 2)["path"] != 3
    assert qplan(4, 2047, 4096, t, 2)["path"] != 3 and qplan(4, 2048, 4096, t, 2)["path"] == 3
    assert qplan(4, 2048, 5120, t, 2)["path"] != 3 and qplan(1, 2048, 8192, t, 2)["path"] != 3
    # 16-bit partials, 2-4 shards: hidden 6144-8192 from 6 rows per CU with 4 wavefronts,
    # otherwise from 3 rows per CU with 8
    assert qplan(2, 2048, 8192, t) == {"path": 3, "waves": 4, "chunks": 4, "grid": 256}
    assert qplan(4, 1535, 8192, t) == {"path": 3, "waves": 8, "chunks": 2, "grid": 256}
    assert qplan(4, 1536, 8192, t)["waves"] == 4 and qplan(4, 767, 8192, t)["path"] != 3
    assert qplan(4, 2048, 6144, t)["waves"] == 4 and qplan(4, 2048, 6136, t)["waves"] == 8
    assert qplan(4, 2048, 4096, t) == {"path": 3, "waves": 8, "chunks": 1, "grid": 256}
    assert qplan(3, 767, 4096, t)["path"] != 3 and qplan(3, 768, 4096, t)["path"] == 3
    assert qplan(1, 2048, 8192, t, 1)["path"] != 3 and qplan(2, 2048, 8192, t, 1)["path"] == 3
    # 5-8 shards from 3 rows per CU, 9-16 from 8, with 8 wavefronts
    assert qplan(5, 2048, 7168, t) == {"path": 3, "waves": 8, "chunks": 2, "grid": 256}
    assert qplan(8, 768, 8192, t)["path"] == 3 and qplan(8, 767, 8192, t)["path"] != 3
    assert qplan(12, 2047, 4096, t)["path"] != 3 and qplan(12, 2048, 4096, t)["waves"] == 8
    # one batch per workgroup, as without a copy
    assert qplan(2, 9 * 256, 8192, t)["path"] == 3 and qplan(2, 9 * 256 + 1, 8192, t)["path"] != 3
    # argument checks
    with pytest.raises(arf.ArfError):
        qplan(4, 2048, 7168, 3)
    with pytest.raises(arf.ArfError):
        qplan(4, 2048, 7176, arf.ARF_QUANT_MXFP4)

def test_plan_claim_region():
    # rows claimed in start order: 4 wavefronts per row, and >= 16 rows per CU with >= 128
    # KiB of traffic per row, or >= 8 rows per CU with >= 256 KiB per row (bf16 8 x 8192:
    # 176 KiB per row; 1 x 16384: exactly 128 KiB; 8 x 16384: 368 KiB)
    assert plan(8, 4095, 8192)["path"] == 2 and plan(8, 4096, 8192)["path"] == 4
    assert plan(1, 4096, 16384)["path"] == 4 and plan(1, 4096, 16376)["path"] == 2
    assert plan(8, 2047, 16384)["path"] == 2 and plan(8, 2048, 16384)["path"] == 4
    # rows of 32-128 KiB from 32 rows per CU, the claims spread over 4 counters (below 96
    # KiB, 4 workgroups per CU) or 2 (2 per CU): 88, 44 and 112 KiB per row
    assert plan(8, 8191, 4096)["path"] == 2
    assert plan(8, 8192, 4096) == {"path": 4, "waves": 4, "chunks": 2, "grid": 8192 + 512}
    assert plan(8, 8192, 2048) == {"path": 4, "waves": 4, "chunks": 1, "grid": 8192 + 512}
    assert plan(4, 8192, 8192) == {"path": 4, "waves": 4, "chunks": 4, "grid": 8192 + 512}
    assert plan(4, 16383, 2048)["path"] == 1            # 28 KiB per row
    assert plan(5, 4096, 7168, 2) == {"path": 4, "waves": 4, "chunks": 4, "grid": 4096 + 256}
    assert plan(8, 8192, 65536)["path"] == 2           # 16 wavefronts
    assert plan(8, 64 * 1024, 16384)["grid"] == 64 * 1024 + 4096
    # the thresholds scale with the CU count
    assert plan(8, 1023, 16384, 0, 128)["path"] == 2 and plan(8, 1024, 16384, 0, 128)["path"] == 4


def test_path_override_forces_and_rejects():
    try:
        arf.arf_set_path_override(1)
        assert plan(8, 8192, 1024)["path"] == 1
        with pytest.raises(arf.ArfError):
            plan(8, 8, 8192)             # a wavefront cannot cover 8192 with 8 chunks/lane
        arf.arf_set_path_override(2, 16, 1)
        assert plan(8, 8, 8192) == {"path": 2, "waves": 16, "chunks": 1, "grid": 8}
        with pytest.raises(arf.ArfError):
            plan(8, 8, 16384)
        arf.arf_set_path_override(3)
        # held rows without a wave count: 8 wavefronts for 16-bit partials, else 4
        assert plan(8, 8192, 16384) == {"path": 3, "waves": 8, "chunks": 4, "grid": 256}
        assert plan(8, 8192, 16384, 2) == {"path": 3, "waves": 4, "chunks": 8, "grid": 256}
        arf.arf_set_path_override(3, 4, 0)
        assert plan(8, 8192, 16384) == {"path": 3, "waves": 4, "chunks": 8, "grid": 256}
        arf.arf_set_path_override(3)
        with pytest.raises(arf.ArfError):
            plan(8, 8, 16392)            # more than 8 chunks per lane
        arf.arf_set_path_override(3, 4, 4)
        assert plan(8, 100, 4096) == {"path": 3, "waves": 4, "chunks": 4, "grid": 100}
        arf.arf_set_path_override(4)     # every row claimed, any size
        # claimants rounded up to a multiple of 8 * split: 4 counters below 96 KiB per row
        assert plan(8, 100, 4096) == {"path": 4, "waves": 4, "chunks": 2, "grid": 192}
        assert plan(8, 8192, 1024)["path"] == 4
        arf.arf_set_path_override(4, 8, 0)
        assert plan(8, 3, 16384) == {"path": 4, "waves": 8, "chunks": 4, "grid": 72}
        for bad in ((5, 0, 0), (0, 4, 0), (2, 3, 0), (2, 2, 0), (2, 4, 3), (1, 8, 0), (3, 16, 0),
                    (4, 2, 0), (4, 4, 3)):
            with pytest.raises(arf.ArfError):
                arf.arf_set_path_override(*bad)
    finally:
        arf.arf_set_path_override(0)
    assert plan(8, 8192, 16384)["waves"] == 4


def test_no_device_returns_hip_error():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake addresses")
    assert call() == HIP
    assert arf.lib().arf_stream_copy(Q, P, 64, None) == HIP


def params(**kw):
    a = dict(n=2, partials=P, tokens=4, row_begin=0, row_count=-1, hidden=64, pdt=0, adt=0,
             acc=0, rin=R, rout=RO, gamma=G, eps=1e-6, nout=NO, q=None, mode=1, sin=None,
             sout=None, size=ctypes.sizeof(arf.arf_params))
    a.update(kw)
    return arf.arf_params(a["size"], a["n"], a["partials"], a["tokens"], a["row_begin"],
                          a["row_count"], a["hidden"], a["pdt"], a["adt"], a["acc"], a["rin"],
                          a["rout"], a["gamma"], a["eps"], a["nout"], a["q"], a["mode"],
                          a["sin"], a["sout"])


def callp(**kw):
    return arf.lib().arf_fused_epilogue(ctypes.byref(params(**kw)), None)


@pytest.mark.parametrize("kw,want", [
    (dict(size=8), VALUE), (dict(acc=2), VALUE), (dict(acc=-1), VALUE),
    (dict(row_begin=-1), SHAPE), (dict(row_begin=5), SHAPE), (dict(row_begin=2, row_count=3), SHAPE),
    (dict(row_begin=4, row_count=0), OK), (dict(row_begin=4), OK), (dict(row_begin=1, row_count=0), OK),
    (dict(partials=None), NULL), (dict(rout=None, nout=None), NOOUT),
    (dict(q=Q, mode=1, sout=None), NULL), (dict(q=Q, mode=3), VALUE), (dict(q=Q, mode=0, sin=None), NULL),
    (dict(q=Q + 8, mode=1, sout=S), ALIGN), (dict(nout=R), ALIAS),
    (dict(tokens=0), OK), (dict(n=0), SHAPE), (dict(adt=2), DTYPE),
])
def test_general_entry_point_validation(kw, want):
    assert callp(**kw) == want


def test_null_params_and_reduce_rows_validation():
    L = arf.lib()
    assert L.arf_fused_epilogue(None, None) == NULL
    rr = L.arf_reduce_rows
    assert rr(P, 2, 4, 0, -1, 64, 0, 0, 0, None, None) == NULL
    assert rr(None, 2, 4, 0, -1, 64, 0, 0, 0, RO, None) == NULL
    assert rr(P, 2, 4, 0, -1, 64, 0, 0, 0, P + 64, None) == ALIAS
    assert rr(P, 2, 4, 3, 2, 64, 0, 0, 0, RO, None) == SHAPE
    assert rr(P, 2, 4, 0, -1, 64, 0, 0, 5, RO, None) == VALUE
    assert rr(P, 2, 4, 0, -1, 64, 1, 0, 0, RO, None) == DTYPE
    assert rr(P, 2, 4, 0, -1, 64, 0, 0, 0, RO + 4, None) == ALIGN
    assert rr(P, 2, 4, 4, -1, 64, 0, 0, 0, None, None) == OK      # empty range
    assert rr(P, 2, 0, 0, -1, 64, 0, 0, 0, None, None) == OK


def test_mxfp4_validation():
    # hidden not a multiple of 32, missing scale buffer, overlap of the block scales
    assert callp(q=Q, mode=2, sout=S, hidden=40) == SHAPE
    assert callp(q=Q, mode=2, sout=None) == NULL
    assert callp(q=Q, mode=2, sout=Q + 64) == ALIAS
    assert callp(q=Q, mode=2, sout=S + 1, tokens=0) == OK
    # the fp8-only entry point does not take the MX mode
    assert callq(mode=2) == VALUE


def test_stream_mix_validation():
    L = arf.lib()
    assert L.arf_stream_mix(None, 0, None, 0, 0, None) == OK
    assert L.arf_stream_mix(Q, 24, P, 32, 0, None) == SHAPE
    assert L.arf_stream_mix(Q, -16, P, 32, 0, None) == SHAPE
    assert L.arf_stream_mix(None, 32, P, 32, 0, None) == NULL
    assert L.arf_stream_mix(Q, 32, None, 32, 0, None) == NULL
    assert L.arf_stream_mix(Q + 8, 32, P, 32, 0, None) == ALIGN
    assert L.arf_stream_mix(P + 16, 64, P, 64, 0, None) == ALIAS
    assert L.arf_stream_mix(Q, 16, P, 16, 2 ** 40, None) == SHAPE


def test_binding_rejects_host_tensors_before_any_call():
    # a host pointer handed to a kernel would fault the GPU: the binding refuses host
    # tensors before it reaches the library
    import torch
    p = torch.zeros((2, 4, 64), dtype=torch.bfloat16)
    r = torch.zeros((4, 64), dtype=torch.bfloat16)
    g = torch.ones((64,), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        arf.arf_reduce_add_rmsnorm(p, r, g, 1e-6, residual_out=r)
    with pytest.raises(ValueError, match="device tensor"):
        arf.arf_reduce_add_rmsnorm_quant(p, r, g, 1e-6, torch.zeros((4, 64), dtype=torch.uint8),
                                         arf.ARF_QUANT_PER_TOKEN)
    with pytest.raises(ValueError, match="device tensor"):
        arf.arf_fused_epilogue(p, r, g, 1e-6, norm_out=r)
    with pytest.raises(ValueError, match="device tensor"):
        arf.arf_reduce_rows(p, r)
    with pytest.raises(ValueError, match=r"\[n_shards\]\[tokens\]\[hidden\]"):
        arf.arf_reduce_rows(p[0], r)
    with pytest.raises(ValueError, match="device tensor"):
        arf.arf_e4m3_encode(torch.zeros(8), torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor"):
        arf.arf_stream_copy(r, r)


def _prototypes():
    """name -> list of parameter declarations, from include/arfuse.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(arf_\w+)\s*\(([^;{]*?)\)\s*;", text):
        params = [p.strip() for p in m.group(2).split(",") if p.strip()]
        out[m.group(1)] = [] if params == ["void"] else params
    return out


def test_binding_signatures_follow_the_header():
    # argument count and pointer-ness of every parameter agree with the C prototypes
    protos = _prototypes()
    assert set(protos) == set(arf.SIGNATURES)
    for name, (res, args) in arf.SIGNATURES.items():
        params = protos[name]
        assert len(params) == len(args), name
        for decl, ct in zip(params, args):
            is_ptr = "*" in decl
            assert is_ptr == (ct is ctypes.c_void_p or ct is ctypes.c_char_p or
                              hasattr(ct, "contents") or ct.__name__.startswith("LP_")), (name, decl)


def test_params_struct_follows_the_header():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct arf_params \{(.*?)\} arf_params;", text, flags=re.S).group(1)
    fields = [l.strip().rstrip(";") for l in body.splitlines() if l.strip()]
    names = [f.split()[-1].lstrip("*") for f in fields]
    assert names == [n for n, _ in arf.arf_params._fields_]
    sizes = {"uint32_t": 4, "int32_t": 4, "int64_t": 8, "float": 4}
    for f, (n, ct) in zip(fields, arf.arf_params._fields_):
        if "*" in f:
            assert ct is ctypes.c_void_p, n
        else:
            assert ctypes.sizeof(ct) == sizes[f.split()[0]], n
