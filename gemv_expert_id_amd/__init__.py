"""Python binding of libmm.so, the gfx950 matrix-product dispatch library.

Argument marshalling only: every entry point below forwards to the C ABI of
the same name (declared in include/mm.h) and every step of the computation
runs in the library's HIP kernels. There is no fallback: if libmm.so is not
built, loading fails with an error.

Buffers are passed as ``Buf(ptr, nbytes)`` (device pointer and the bytes
valid from it); ``buf(tensor)`` builds one from a torch tensor. ``stream`` is
a hipStream_t handle as an int (``torch.cuda.current_stream().cuda_stream``),
a torch stream object, or None for the null stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmm.so")

MM_F32, MM_F16, MM_BF16 = 0, 1, 2
MM_ROUTE_GEMV, MM_ROUTE_GEMM, MM_ROUTE_ID_DIRECT = 0, 1, 2
MM_ROUTE_ID_MAP, MM_ROUTE_ID_GROUPED, MM_ROUTE_ID_PREFILL = 3, 4, 5
MM_ROUTE_GEMV_WIDE = 6
# mm_kernel: kernel family reported in receipts
(MM_KERNEL_GEMV_ROWS, MM_KERNEL_GEMV_ROWS_ELEM, MM_KERNEL_GEMV_COLS, MM_KERNEL_GEMM_TILED,
 MM_KERNEL_GEMM_LARGE, MM_KERNEL_GEMM_F32, MM_KERNEL_ID_DIRECT_FAST, MM_KERNEL_ID_DIRECT,
 MM_KERNEL_ID_MAP, MM_KERNEL_ID_GROUPED_MFMA, MM_KERNEL_ID_GROUPED_FMA,
 MM_KERNEL_GEMV_WIDE, MM_KERNEL_GEMM_F32_SMALL, MM_KERNEL_GEMM_PANEL) = range(14)
MM_ID_SCHEMA_VERSION = 5
MM_ID_GROUPED_MAX_EXPERTS = 1024

STATUS_NAMES = {
    0: "MM_OK", 1: "MM_ERR_INVALID_ARGUMENT", 2: "MM_ERR_UNSUPPORTED",
    3: "MM_ERR_BUFFER_TOO_SMALL", 4: "MM_ERR_MISALIGNED", 5: "MM_ERR_OVERLAP",
    6: "MM_ERR_SCRATCH", 7: "MM_ERR_DEVICE",
}

# Every symbol include/mm.h declares.
EXPORTS = [
    "mm_gemm", "mm_gemm_ex", "mm_gemm_route", "mm_gemv", "mm_id_query", "mm_id_route_hint", "mm_id_direct", "mm_id_map",
    "mm_id_grouped",
    "mm_id", "mm_capabilities", "mm_status_string", "mm_last_error",
    "mm_test_inject_resolve_failure", "mm_test_launch_count", "mm_id_prefill_noalloc",
]
MM_ID_NOALLOC_SCRATCH_BYTES = 4 << 20


class MmError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


class Buf(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("bytes", ctypes.c_uint64)]


class Receipt(ctypes.Structure):
    _fields_ = [("schema_version", ctypes.c_uint32), ("route", ctypes.c_uint32),
                ("dtype", ctypes.c_uint32), ("dispatch_count", ctypes.c_uint32),
                ("kernel", ctypes.c_uint32), ("variant", ctypes.c_uint32)]


class GemmDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("trans_a", ctypes.c_int32), ("trans_b", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("m", ctypes.c_int64), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64),
                ("ldc", ctypes.c_int64), ("stride_a", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_c", ctypes.c_int64),
                ("offset_a", ctypes.c_uint64), ("offset_b", ctypes.c_uint64),
                ("offset_c", ctypes.c_uint64)]


class IdParams(ctypes.Structure):
    _fields_ = [("m", ctypes.c_uint32), ("n", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("top_k", ctypes.c_uint32), ("n_experts", ctypes.c_uint32),
                ("expert_stride_bytes", ctypes.c_uint64), ("input_layout", ctypes.c_uint32),
                ("multiplicity", ctypes.c_uint32), ("route", ctypes.c_uint32)]


class IdCapability(ctypes.Structure):
    _fields_ = [("schema_version", ctypes.c_uint32), ("weight_dtype", ctypes.c_uint32),
                ("route", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("weight_bytes", ctypes.c_uint64), ("input_bytes", ctypes.c_uint64),
                ("ids_bytes", ctypes.c_uint64), ("output_bytes", ctypes.c_uint64),
                ("counts_bytes", ctypes.c_uint64), ("routed_rows_bytes", ctypes.c_uint64)]


class DeviceCaps(ctypes.Structure):
    _fields_ = [("arch", ctypes.c_char * 64), ("cu_count", ctypes.c_int32),
                ("max_clock_mhz", ctypes.c_int32), ("l2_bytes", ctypes.c_int32),
                ("xcd_count", ctypes.c_int32), ("hbm_bytes", ctypes.c_uint64),
                ("dtype_mask", ctypes.c_uint32), ("max_grouped_experts", ctypes.c_uint32),
                ("abi_version", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmm.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gemv_expert_id_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    st = ctypes.c_int
    vp = ctypes.c_void_p
    lib.mm_gemm.argtypes = [P(GemmDesc), Buf, Buf, Buf, vp, P(Receipt)]
    lib.mm_gemm.restype = st
    lib.mm_gemm_ex.argtypes = [P(GemmDesc), ctypes.c_float, ctypes.c_float, Buf, Buf, Buf, vp,
                               P(Receipt)]
    lib.mm_gemm_ex.restype = st
    lib.mm_gemm_route.argtypes = [P(GemmDesc), ctypes.c_uint32, ctypes.c_float, ctypes.c_float,
                                  Buf, Buf, Buf, vp, P(Receipt)]
    lib.mm_gemm_route.restype = st
    lib.mm_gemv.argtypes = [P(GemmDesc), Buf, Buf, Buf, vp, P(Receipt)]
    lib.mm_gemv.restype = st
    lib.mm_id_query.argtypes = [ctypes.c_int, P(IdParams), P(IdCapability)]
    lib.mm_id_query.restype = st
    lib.mm_id_route_hint.argtypes = [ctypes.c_int, P(IdParams), P(ctypes.c_uint32)]
    lib.mm_id_route_hint.restype = st
    lib.mm_id_direct.argtypes = [P(IdParams), ctypes.c_int, Buf, Buf, Buf, Buf, vp, P(Receipt)]
    lib.mm_id_direct.restype = st
    lib.mm_id_map.argtypes = [P(IdParams), Buf, Buf, Buf, Buf, vp, P(Receipt)]
    lib.mm_id_map.restype = st
    lib.mm_id_grouped.argtypes = [P(IdParams), ctypes.c_int, Buf, Buf, Buf, Buf, Buf, vp,
                                  P(Receipt)]
    lib.mm_id_grouped.restype = st
    lib.mm_id.argtypes = [P(IdParams), ctypes.c_int, Buf, Buf, Buf, Buf, Buf, Buf, vp,
                          P(Receipt)]
    lib.mm_id.restype = st
    lib.mm_id_prefill_noalloc.argtypes = [P(IdParams), ctypes.c_int, Buf, Buf, Buf, Buf, vp,
                                          P(Receipt)]
    lib.mm_id_prefill_noalloc.restype = st
    lib.mm_capabilities.argtypes = [ctypes.c_int, P(DeviceCaps)]
    lib.mm_capabilities.restype = st
    lib.mm_status_string.argtypes = [ctypes.c_int]
    lib.mm_status_string.restype = ctypes.c_char_p
    lib.mm_last_error.argtypes = []
    lib.mm_last_error.restype = ctypes.c_char_p
    lib.mm_test_inject_resolve_failure.argtypes = [ctypes.c_char_p]
    lib.mm_test_inject_resolve_failure.restype = None
    lib.mm_test_launch_count.argtypes = []
    lib.mm_test_launch_count.restype = ctypes.c_uint64
    _lib = lib
    return lib


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        return ctypes.c_void_p(0)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _raise(status: int):
    if status != 0:
        raise MmError(status, load().mm_last_error().decode())


def buf(t, nbytes: Optional[int] = None) -> Buf:
    """Buf for a torch tensor (or anything with data_ptr/numel/element_size)."""
    if t is None:
        return Buf(None, 0)
    n = t.numel() * t.element_size() if nbytes is None else nbytes
    return Buf(t.data_ptr(), n)


def gemm_desc(dtype: int, m: int, n: int, k: int, *, batch: int = 1, trans_a: bool = False,
              trans_b: bool = False, lda: int = 0, ldb: int = 0, ldc: int = 0,
              stride_a: int = 0, stride_b: int = 0, stride_c: int = 0, offset_a: int = 0,
              offset_b: int = 0, offset_c: int = 0) -> GemmDesc:
    return GemmDesc(dtype, int(trans_a), int(trans_b), batch, m, n, k, lda, ldb, ldc, stride_a,
                    stride_b, stride_c, offset_a, offset_b, offset_c)


def id_params(m: int, n: int, k: int, top_k: int, n_experts: int, expert_stride_bytes: int,
              input_layout: int = 0, multiplicity: int = 0, route: int = 0) -> IdParams:
    return IdParams(m, n, k, top_k, n_experts, expert_stride_bytes, input_layout, multiplicity,
                    route)


def mm_gemm(desc: GemmDesc, a: Buf, b: Buf, c: Buf, stream=None) -> Receipt:
    r = Receipt()
    _raise(load().mm_gemm(ctypes.byref(desc), a, b, c, _stream(stream), ctypes.byref(r)))
    return r


def mm_gemm_ex(desc: GemmDesc, alpha: float, beta: float, a: Buf, b: Buf, c: Buf,
               stream=None) -> Receipt:
    """C = alpha * op(A) op(B) + beta * C (beta == 0: old C unread)."""
    r = Receipt()
    _raise(load().mm_gemm_ex(ctypes.byref(desc), ctypes.c_float(alpha), ctypes.c_float(beta),
                             a, b, c, _stream(stream), ctypes.byref(r)))
    return r


def mm_gemm_route(desc: GemmDesc, route: int, a: Buf, b: Buf, c: Buf, alpha: float = 1.0,
                  beta: float = 0.0, stream=None) -> Receipt:
    """The product on the route the caller names (GEMV, skinny or tiled GEMM)."""
    r = Receipt()
    _raise(load().mm_gemm_route(ctypes.byref(desc), route, ctypes.c_float(alpha),
                                ctypes.c_float(beta), a, b, c, _stream(stream), ctypes.byref(r)))
    return r


def mm_gemv(desc: GemmDesc, a: Buf, b: Buf, c: Buf, stream=None) -> Receipt:
    r = Receipt()
    _raise(load().mm_gemv(ctypes.byref(desc), a, b, c, _stream(stream), ctypes.byref(r)))
    return r


def mm_id_query(weight_dtype: int, params: IdParams) -> IdCapability:
    cap = IdCapability()
    _raise(load().mm_id_query(weight_dtype, ctypes.byref(params), ctypes.byref(cap)))
    return cap


def mm_id_route_hint(weight_dtype: int, params: IdParams) -> int:
    """0 (direct) or 1 (grouped prefill): the route measured faster for this problem."""
    r = ctypes.c_uint32(0)
    _raise(load().mm_id_route_hint(weight_dtype, ctypes.byref(params), ctypes.byref(r)))
    return int(r.value)


def mm_id_direct(params: IdParams, weight_dtype: int, weights: Buf, inp: Buf, ids: Buf,
                 out: Buf, stream=None) -> Receipt:
    r = Receipt()
    _raise(load().mm_id_direct(ctypes.byref(params), weight_dtype, weights, inp, ids, out,
                               _stream(stream), ctypes.byref(r)))
    return r


def mm_id_map(params: IdParams, ids: Buf, counts: Buf, routed_rows: Buf, out: Buf,
              stream=None) -> Receipt:
    r = Receipt()
    _raise(load().mm_id_map(ctypes.byref(params), ids, counts, routed_rows, out,
                            _stream(stream), ctypes.byref(r)))
    return r


def mm_id_grouped(params: IdParams, weight_dtype: int, weights: Buf, inp: Buf, counts: Buf,
                  routed_rows: Buf, out: Buf, stream=None) -> Receipt:
    r = Receipt()
    _raise(load().mm_id_grouped(ctypes.byref(params), weight_dtype, weights, inp, counts,
                                routed_rows, out, _stream(stream), ctypes.byref(r)))
    return r


def mm_id(params: IdParams, weight_dtype: int, weights: Buf, inp: Buf, ids: Buf, out: Buf,
          counts: Optional[Buf] = None, routed_rows: Optional[Buf] = None,
          stream=None) -> Receipt:
    r = Receipt()
    _raise(load().mm_id(ctypes.byref(params), weight_dtype, weights, inp, ids, out,
                        counts or Buf(None, 0), routed_rows or Buf(None, 0), _stream(stream),
                        ctypes.byref(r)))
    return r


def mm_id_prefill_noalloc(params: IdParams, weight_dtype: int, weights: Buf, inp: Buf, ids: Buf,
                          out: Buf, stream=None) -> Receipt:
    """Map + grouped prefill with the library's own scratch (no allocation)."""
    r = Receipt()
    _raise(load().mm_id_prefill_noalloc(ctypes.byref(params), weight_dtype, weights, inp, ids,
                                        out, _stream(stream), ctypes.byref(r)))
    return r


def mm_capabilities(device: int = 0) -> DeviceCaps:
    caps = DeviceCaps()
    _raise(load().mm_capabilities(device, ctypes.byref(caps)))
    return caps


def mm_status_string(status: int) -> str:
    return load().mm_status_string(status).decode()


def mm_last_error() -> str:
    return load().mm_last_error().decode()
