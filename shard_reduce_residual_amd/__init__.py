"""Python binding of libarfuse (argument marshalling only).

Every step of the fused reduce + residual + RMSNorm (+fp8) path runs in the HIP
kernels of ``libarfuse.so``; this module only turns torch tensors into device pointers,
sizes and a stream handle, calls the C ABI declared in ``include/arfuse.h`` and turns a
non-zero status into an exception. There is no fallback: if the library is missing the
import of a function raises.
"""
from __future__ import annotations

import ctypes
import glob
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libarfuse.so")

ARF_BF16, ARF_F16, ARF_F32 = 0, 1, 2
ARF_QUANT_NONE, ARF_QUANT_PER_TENSOR, ARF_QUANT_PER_TOKEN, ARF_QUANT_MXFP4 = -1, 0, 1, 2
ARF_ACC_F32, ARF_ACC_PARTIAL = 0, 1
ARF_MAX_SHARDS, ARF_MAX_HIDDEN = 16, 65536
STATUS = ["ARF_OK", "ARF_ERR_NULL", "ARF_ERR_SHAPE", "ARF_ERR_DTYPE", "ARF_ERR_ALIGN",
          "ARF_ERR_ALIAS", "ARF_ERR_NO_OUTPUT", "ARF_ERR_VALUE", "ARF_ERR_HIP"]

_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class arf_params(ctypes.Structure):
    """Mirror of ``arf_params`` in include/arfuse.h."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("n_shards", _i32), ("partials", _vp),
                ("tokens", _i64), ("row_begin", _i64), ("row_count", _i64),
                ("hidden", _i32), ("partial_dtype", _i32), ("act_dtype", _i32),
                ("accumulate", _i32), ("residual_in", _vp), ("residual_out", _vp),
                ("gamma", _vp), ("eps", _f32), ("norm_out", _vp), ("quant_out", _vp),
                ("quant_mode", _i32), ("scale_in", _vp), ("scale_out", _vp)]


# Exported symbols and their C signatures (kept in step with include/arfuse.h).
SIGNATURES = {
    "arf_reduce_add_rmsnorm": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _f32,
                                      _vp, _vp]),
    "arf_reduce_add_rmsnorm_quant": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp,
                                            _f32, _vp, _vp, _i32, _vp, _vp, _vp]),
    "arf_fused_epilogue": (_i32, [ctypes.POINTER(arf_params), _vp]),
    "arf_reduce_rows": (_i32, [_vp, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp]),
    "arf_status_string": (ctypes.c_char_p, [_i32]),
    "arf_version": (_i32, []),
    "arf_get_plan": (_i32, [_i32, _i64, _i32, _i32, _i32, ctypes.POINTER(_i32)]),
    "arf_get_plan_quant": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32)]),
    "arf_set_path_override": (_i32, [_i32, _i32, _i32]),
    "arf_e4m3_encode": (_i32, [_vp, _vp, _i64, _vp]),
    "arf_e2m1_encode": (_i32, [_vp, _vp, _i64, _vp]),
    "arf_stream_copy": (_i32, [_vp, _vp, _i64, _vp]),
    "arf_stream_mix": (_i32, [_vp, _i64, _vp, _i64, _i64, _vp]),
}


class ArfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__("%s returned %s" % (where, name))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libarfuse.so (built by ``shard_reduce_residual_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libarfuse.so is not built (%s); run "
                              "`python -m shard_reduce_residual_amd.build`" % LIB_PATH)
        built = os.path.getmtime(LIB_PATH)
        newer = [f for f in glob.glob(os.path.join(HERE, "csrc", "*")) +
                 [os.path.join(os.path.dirname(HERE), "include", "arfuse.h")]
                 if os.path.exists(f) and os.path.getmtime(f) > built]
        if newer:
            sys.stderr.write("warning: libarfuse.so is older than %s; rebuild with "
                             "`python -m shard_reduce_residual_amd.build`\n"
                             % ", ".join(os.path.basename(f) for f in newer))
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


_T = None


def _types():
    """torch dtypes used by the checks, resolved once (torch is imported lazily)."""
    global _T
    if _T is None:
        import torch

        class _Types:
            codes = {torch.bfloat16: ARF_BF16, torch.float16: ARF_F16, torch.float32: ARF_F32}
            act = (torch.bfloat16, torch.float16)
            f32 = (torch.float32,)
            u8 = (torch.uint8,)
        _T = _Types
    return _T


def _dtype_code(t) -> int:
    code = _types().codes.get(t.dtype)
    if code is None:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return code


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _dev(name, t, dev, numel=None, dtypes=None):
    """Device pointer of ``t`` after the checks the C ABI cannot make: a contiguous tensor
    on device index ``dev`` (a host pointer handed to a kernel would fault the GPU), with
    ``numel`` elements of one of ``dtypes`` (a short buffer would be written past its end).
    None stays None (an optional buffer left out)."""
    if t is None:
        return None
    if (t.get_device() == dev and (numel is None or t.numel() == numel)
            and (dtypes is None or t.dtype in dtypes) and t.is_contiguous()):
        return t.data_ptr()
    if t.get_device() != dev:
        raise ValueError("%s is on %s; the call runs on cuda:%d" % (name, t.device, dev))
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s; expected %s" % (name, t.dtype, dtypes))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements; expected %d" % (name, t.numel(), numel))
    raise ValueError("%s must be contiguous" % name)


def _partials(partials):
    """(n_shards, tokens, hidden, device index) of a [N][T][H] device tensor."""
    dev = partials.get_device()
    if partials.dim() != 3:
        raise ValueError("partials must be [n_shards][tokens][hidden]")
    if dev < 0:
        raise ValueError("partials must be a device tensor (got %s)" % partials.device)
    n, t, h = partials.shape
    return n, t, h, dev


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, where: str):
    if st != 0:
        raise ArfError(st, where)


def arf_reduce_add_rmsnorm(partials, residual_in, gamma, eps: float, residual_out=None,
                           norm_out=None, stream=None) -> None:
    """partials [N][T][H] (bf16/f16, or f32); residual_in/_out, norm_out [T][H] and
    gamma [H] in the activation type. Enqueues one kernel on ``stream``."""
    n, t, h, dev = _partials(partials)
    act = (residual_in.dtype,)
    st = lib().arf_reduce_add_rmsnorm(_ptr(partials), n, t, h, _dtype_code(partials),
                                      _dtype_code(residual_in),
                                      _dev("residual_in", residual_in, dev, t * h, _types().act),
                                      _dev("residual_out", residual_out, dev, t * h, act),
                                      _dev("gamma", gamma, dev, h, act), float(eps),
                                      _dev("norm_out", norm_out, dev, t * h, act),
                                      _stream(stream))
    _check(st, "arf_reduce_add_rmsnorm")


def arf_reduce_add_rmsnorm_quant(partials, residual_in, gamma, eps: float, quant_out,
                                 mode: int, scale_in=None, scale_out=None,
                                 residual_out=None, norm_out=None, stream=None) -> None:
    """As arf_reduce_add_rmsnorm plus ``quant_out`` [T][H] uint8 E4M3 codes;
    ``mode`` ARF_QUANT_PER_TENSOR (``scale_in``: 1-element f32 device tensor) or
    ARF_QUANT_PER_TOKEN (``scale_out``: [T] f32 device tensor, written)."""
    n, t, h, dev = _partials(partials)
    act, T = (residual_in.dtype,), _types()
    st = lib().arf_reduce_add_rmsnorm_quant(
        _ptr(partials), n, t, h, _dtype_code(partials), _dtype_code(residual_in),
        _dev("residual_in", residual_in, dev, t * h, T.act),
        _dev("residual_out", residual_out, dev, t * h, act),
        _dev("gamma", gamma, dev, h, act), float(eps),
        _dev("norm_out", norm_out, dev, t * h, act),
        _dev("quant_out", quant_out, dev, t * h, T.u8), int(mode),
        _dev("scale_in", scale_in, dev, 1, T.f32),
        _dev("scale_out", scale_out, dev, t, T.f32), _stream(stream))
    _check(st, "arf_reduce_add_rmsnorm_quant")


def arf_fused_epilogue(partials, residual_in, gamma, eps: float, residual_out=None,
                       norm_out=None, quant_out=None, mode: int = ARF_QUANT_PER_TOKEN,
                       scale_in=None, scale_out=None, accumulate: int = ARF_ACC_F32,
                       row_begin: int = 0, row_count: int = -1, stream=None) -> None:
    """The general call: row range and accumulation mode (see arf_params)."""
    n, t, h, dev = _partials(partials)
    act, T = (residual_in.dtype,), _types()
    mx = quant_out is not None and mode == ARF_QUANT_MXFP4
    a = arf_params(ctypes.sizeof(arf_params), n, _ptr(partials), t, row_begin, row_count, h,
                   _dtype_code(partials), _dtype_code(residual_in), accumulate,
                   _dev("residual_in", residual_in, dev, t * h, T.act),
                   _dev("residual_out", residual_out, dev, t * h, act),
                   _dev("gamma", gamma, dev, h, act), float(eps),
                   _dev("norm_out", norm_out, dev, t * h, act),
                   _dev("quant_out", quant_out, dev, t * h // 2 if mx else t * h, T.u8), mode,
                   _dev("scale_in", scale_in, dev, 1, T.f32),
                   _dev("scale_out", scale_out, dev, t * h // 32 if mx else t,
                        T.u8 if mx else T.f32))
    _check(lib().arf_fused_epilogue(ctypes.byref(a), _stream(stream)), "arf_fused_epilogue")


def arf_reduce_rows(partials, sums_out, row_begin: int = 0, row_count: int = -1,
                    accumulate: int = ARF_ACC_F32, stream=None) -> None:
    """Reduced values of rows [row_begin, row_begin + row_count) into sums_out [T][H]."""
    n, t, h, dev = _partials(partials)
    _check(lib().arf_reduce_rows(_ptr(partials), n, t, row_begin, row_count, h,
                                 _dtype_code(partials), _dtype_code(sums_out), accumulate,
                                 _dev("sums_out", sums_out, dev, t * h, _types().act),
                                 _stream(stream)), "arf_reduce_rows")


def arf_status_string(status: int) -> str:
    return lib().arf_status_string(status).decode()


def arf_version() -> int:
    return lib().arf_version()


def arf_get_plan(n_shards: int, tokens: int, hidden: int, partial_dtype: int,
                 num_cus: int = 0) -> dict:
    out = (_i32 * 4)()
    _check(lib().arf_get_plan(n_shards, tokens, hidden, partial_dtype, num_cus, out),
           "arf_get_plan")
    return {"path": out[0], "waves": out[1], "chunks": out[2], "grid": out[3]}


def arf_get_plan_quant(n_shards: int, tokens: int, hidden: int, partial_dtype: int,
                       quant_mode: int, num_cus: int = 0) -> dict:
    out = (_i32 * 4)()
    _check(lib().arf_get_plan_quant(n_shards, tokens, hidden, partial_dtype, quant_mode,
                                    num_cus, out), "arf_get_plan_quant")
    return {"path": out[0], "waves": out[1], "chunks": out[2], "grid": out[3]}


def arf_set_path_override(path: int, waves_per_block: int = 0, chunks_per_lane: int = 0):
    _check(lib().arf_set_path_override(path, waves_per_block, chunks_per_lane),
           "arf_set_path_override")


def arf_e4m3_encode(x, out, stream=None) -> None:
    dev = x.get_device()
    if dev < 0:
        raise ValueError("x must be a device tensor (got %s)" % x.device)
    _check(lib().arf_e4m3_encode(_dev("x", x, dev, None, _types().f32),
                                 _dev("out", out, dev, x.numel(), _types().u8),
                                 x.numel(), _stream(stream)), "arf_e4m3_encode")


def arf_e2m1_encode(x, out, stream=None) -> None:
    dev = x.get_device()
    if dev < 0:
        raise ValueError("x must be a device tensor (got %s)" % x.device)
    _check(lib().arf_e2m1_encode(_dev("x", x, dev, None, _types().f32),
                                 _dev("out", out, dev, x.numel(), _types().u8),
                                 x.numel(), _stream(stream)), "arf_e2m1_encode")


def _bytes_at_least(name, t, nbytes):
    if t.get_device() < 0:
        raise ValueError("%s must be a device tensor (got %s)" % (name, t.device))
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes; %d are accessed"
                         % (name, t.numel() * t.element_size(), nbytes))
    return _ptr(t)


def arf_stream_copy(dst, src, nbytes: int | None = None, stream=None) -> None:
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().arf_stream_copy(_bytes_at_least("dst", dst, nbytes),
                                 _bytes_at_least("src", src, nbytes), nbytes, _stream(stream)),
           "arf_stream_copy")


def arf_stream_mix(dst, write_bytes: int, src, read_bytes: int, units: int = 0,
                   stream=None) -> None:
    _check(lib().arf_stream_mix(_bytes_at_least("dst", dst, write_bytes) if write_bytes else None,
                                write_bytes,
                                _bytes_at_least("src", src, read_bytes) if read_bytes else None,
                                read_bytes, units, _stream(stream)), "arf_stream_mix")
