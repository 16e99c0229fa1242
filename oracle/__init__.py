"""Oracle for the fused reduce + residual + RMSNorm (+fp8-e4m3) epilogue.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product library never
loads it, and it shares no code with the HIP path.

The arithmetic lives in ``arf_oracle.c`` (plain scalar C, threaded over rows). This
module compiles it with gcc when the shared object is missing or older than the source,
and marshals numpy arrays to it. 16-bit element types travel as ``np.uint16`` bit
patterns; fp32 partials as ``np.float32``.

Method: TensorRT-LLM page "allReduceFusionKernels.cu" (allreduce_sum, add128,
rms_norm, fused_op, oneshot-sync post-barrier loop); FlashInfer page for
trtllm_create_ipc_workspace_for_all_reduce_fusion (buffer shape, fp32 partials);
OCP OFP8 rev 1.0 (E4M3); OCP Microscaling Formats v1.0 (MXFP4).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "arf_oracle.c")
_LIB = os.path.join(_HERE, "libarf_oracle.so")

DTYPES = {"bf16": 0, "f16": 1, "f32": 2}
MODES = {"per_tensor": 0, "per_token": 1, "mxfp4": 2}
ACCUMULATE = {"f32": 0, "partial": 1}


class Args(ctypes.Structure):
    """Mirror of ``arfo_args`` in arf_oracle.h."""
    _fields_ = [("partials", ctypes.c_void_p), ("n_shards", ctypes.c_int32),
                ("tokens", ctypes.c_int64), ("hidden", ctypes.c_int32),
                ("partial_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("accumulate", ctypes.c_int32), ("row_begin", ctypes.c_int64),
                ("row_count", ctypes.c_int64), ("residual_in", ctypes.c_void_p),
                ("residual_out", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("norm_out", ctypes.c_void_p),
                ("quant_out", ctypes.c_void_p), ("quant_mode", ctypes.c_int32),
                ("scale_in", ctypes.c_void_p), ("scale_out", ctypes.c_void_p),
                ("n_threads", ctypes.c_int32)]


def build(force: bool = False) -> str:
    """Compile the oracle into ``oracle/libarf_oracle.so`` and return its path."""
    header = os.path.join(os.path.dirname(_SRC), "arf_oracle.h")
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= max(os.path.getmtime(_SRC), os.path.getmtime(header))):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.arfo_f32_to_bf16.argtypes = [f32]
        L.arfo_f32_to_bf16.restype = ctypes.c_uint16
        L.arfo_f32_to_f16.argtypes = [f32]
        L.arfo_f32_to_f16.restype = ctypes.c_uint16
        L.arfo_f32_to_e4m3.argtypes = [f32]
        L.arfo_f32_to_e4m3.restype = ctypes.c_uint8
        L.arfo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.arfo_bf16_to_f32.restype = f32
        L.arfo_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.arfo_f16_to_f32.restype = f32
        L.arfo_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.arfo_e4m3_to_f32.restype = f32
        L.arfo_f32_to_e2m1.argtypes = [f32]
        L.arfo_f32_to_e2m1.restype = ctypes.c_uint8
        L.arfo_e2m1_to_f32.argtypes = [ctypes.c_uint8]
        L.arfo_e2m1_to_f32.restype = f32
        L.arfo_mx_scale_code.argtypes = [f32]
        L.arfo_mx_scale_code.restype = ctypes.c_uint8
        for name in ("arfo_f32_to_bf16_n", "arfo_f32_to_f16_n", "arfo_f32_to_e4m3_n",
                     "arfo_f32_to_e2m1_n"):
            getattr(L, name).argtypes = [vp, vp, i64]
            getattr(L, name).restype = None
        L.arfo_reduce_add_rmsnorm.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp, f32,
                                              vp, i32]
        L.arfo_reduce_add_rmsnorm.restype = ctypes.c_int
        L.arfo_reduce_add_rmsnorm_quant.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp,
                                                    f32, vp, vp, i32, vp, vp, i32]
        L.arfo_reduce_add_rmsnorm_quant.restype = ctypes.c_int
        L.arfo_run.argtypes = [ctypes.POINTER(Args)]
        L.arfo_run.restype = ctypes.c_int
        L.arfo_reduce_rows.argtypes = [vp, i32, i64, i32, i32, i32, i32, i64, i64, vp, i32]
        L.arfo_reduce_rows.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---- scalar / bulk conversions -----------------------------------------------------

def f32_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().arfo_f32_to_bf16_n(_ptr(x), _ptr(out), x.size)
    return out


def f32_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().arfo_f32_to_f16_n(_ptr(x), _ptr(out), x.size)
    return out


def f32_to_e4m3(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().arfo_f32_to_e4m3_n(_ptr(x), _ptr(out), x.size)
    return out


def f32_to_e2m1(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().arfo_f32_to_e2m1_n(_ptr(x), _ptr(out), x.size)
    return out


def mx_scale_code(amax) -> np.ndarray:
    f = lib().arfo_mx_scale_code
    a = np.ascontiguousarray(amax, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], np.uint8).reshape(a.shape)


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f16_to_f32(h) -> np.ndarray:
    f = lib().arfo_f16_to_f32
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return np.array([f(int(v)) for v in h.ravel()], np.float32).reshape(h.shape)


def e4m3_to_f32(q) -> np.ndarray:
    f = lib().arfo_e4m3_to_f32
    q = np.ascontiguousarray(q, dtype=np.uint8)
    return np.array([f(int(v)) for v in q.ravel()], np.float32).reshape(q.shape)


def act_to_f32(bits, act: str) -> np.ndarray:
    return bf16_to_f32(bits) if act == "bf16" else f16_to_f32(bits)


# ---- the fused epilogue ---------------------------------------------------------------

class OracleError(RuntimeError):
    pass


def reduce_add_rmsnorm(partials: np.ndarray, residual_in: np.ndarray, gamma: np.ndarray,
                       eps: float, *, partial_dtype: str, act_dtype: str,
                       residual_out: bool = True, norm_out: bool = True,
                       quant: str | None = None, scale_in: float | None = None,
                       residual_out_array: np.ndarray | None = None,
                       accumulate: str = "f32", rows: tuple | None = None,
                       out_init: int | None = None,
                       n_threads: int | None = None) -> dict:
    """Run the oracle. ``partials`` is [N][T][H] (uint16 bits or float32),
    ``residual_in`` [T][H] uint16 bits, ``gamma`` [H] uint16 bits.

    Returns a dict with ``residual_out`` / ``norm_out`` (uint16 bits), ``quant_out``
    (uint8 codes; "mxfp4": [T][H/2], two E2M1 codes per byte, even element in the low
    nibble) and ``scale_out`` (float32 [T] for "per_token"; uint8 E8M0 [T][H/32] for
    "mxfp4") as requested.
    ``residual_out_array`` may be ``residual_in`` itself to run in place. ``accumulate``
    is "f32" (the default branch) or "partial" (rounded to the partial type after every
    addition). ``rows`` = (begin, count) restricts the computed rows; output rows outside
    it keep ``out_init`` (a byte value, default 0).
    """
    n, t, h = partials.shape
    want_p = np.float32 if partial_dtype == "f32" else np.uint16
    partials = np.ascontiguousarray(partials, dtype=want_p)
    if residual_out_array is None:
        residual_in = np.ascontiguousarray(residual_in, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    assert residual_in.shape == (t, h) and gamma.shape == (h,)
    fill = 0 if out_init is None else out_init

    def new(shape, dtype):
        a = np.empty(shape, dtype)
        a.view(np.uint8)[...] = fill
        return a

    out = {}
    if residual_out_array is not None:
        rout = residual_out_array
        out["residual_out"] = rout
    else:
        rout = new((t, h), np.uint16) if residual_out else None
        if rout is not None:
            out["residual_out"] = rout
    nout = new((t, h), np.uint16) if norm_out else None
    if nout is not None:
        out["norm_out"] = nout
    thr = default_threads() if n_threads is None else n_threads
    q = sin = sout = None
    mode = -1
    if quant is not None:
        mode = MODES[quant]
        if quant == "mxfp4":
            q = new((t, h // 2), np.uint8)
            sout = new((t, h // 32), np.uint8)
        else:
            q = new((t, h), np.uint8)
        out["quant_out"] = q
        if quant == "per_tensor":
            sin = np.array([scale_in], np.float32)
        elif quant == "per_token":
            sout = new((t,), np.float32)
        if sout is not None:
            out["scale_out"] = sout
    begin, count = (0, -1) if rows is None else rows
    a = Args(_ptr(partials), n, t, h, DTYPES[partial_dtype], DTYPES[act_dtype],
             ACCUMULATE[accumulate], begin, count, _ptr(residual_in), _ptr(rout), _ptr(gamma),
             eps, _ptr(nout), _ptr(q), mode, _ptr(sin), _ptr(sout), thr)
    rc = lib().arfo_run(ctypes.byref(a))
    if rc != 0:
        raise OracleError("oracle rejected the arguments (code %d)" % rc)
    return out


def reduce_rows(partials: np.ndarray, *, partial_dtype: str, act_dtype: str,
                accumulate: str = "f32", rows: tuple | None = None,
                out_init: int = 0, n_threads: int | None = None) -> np.ndarray:
    """The reduced value (cast to the activation type) of rows (begin, count) of
    [N][T][H] partials, as a [T][H] uint16 array; other rows keep ``out_init`` bytes."""
    n, t, h = partials.shape
    want_p = np.float32 if partial_dtype == "f32" else np.uint16
    partials = np.ascontiguousarray(partials, dtype=want_p)
    sums = np.empty((t, h), np.uint16)
    sums.view(np.uint8)[...] = out_init
    begin, count = (0, -1) if rows is None else rows
    thr = default_threads() if n_threads is None else n_threads
    rc = lib().arfo_reduce_rows(_ptr(partials), n, t, h, DTYPES[partial_dtype],
                                DTYPES[act_dtype], ACCUMULATE[accumulate], begin, count,
                                _ptr(sums), thr)
    if rc != 0:
        raise OracleError("oracle rejected the arguments (code %d)" % rc)
    return sums
