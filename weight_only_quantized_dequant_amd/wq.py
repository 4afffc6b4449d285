"""Python binding of libwq: the C ABI of include/wq.h under the same names.

Argument marshalling only. Every step of the path, including quantize and pack, runs
inside libwq.so (host C++ or HIP kernels). Host arrays are numpy arrays. Device
buffers are torch tensors, which serve only as device memory and streams. A missing
library raises an error; there is no fallback.
"""

import ctypes
import os

import numpy as np

FMT_F16, FMT_W8, FMT_W4G32, FMT_W6E3M2, FMT_W4E2M1, FMT_BF16, FMT_W5E2M2 = 0, 1, 2, 3, 4, 5, 6
FMT_NAMES = {"f16": FMT_F16, "w8": FMT_W8, "w4g32": FMT_W4G32, "w6e3m2": FMT_W6E3M2, "w4e2m1": FMT_W4E2M1,
             "bf16": FMT_BF16, "w5e2m2": FMT_W5E2M2}
# OR-ed into a format code: bfloat16 activations (x, y and dequantized weights) instead of fp16
ACT_F16, ACT_BF16 = 0, 0x100

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class LinearItem(ctypes.Structure):
    """wq_linear_item: one linear of a grouped call (device pointers)."""
    _fields_ = [("x", ctypes.c_void_p), ("packed_w", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class WqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        text = lib().wq_status_string(status).decode()
        if status == -6:
            text += " [%s]" % lib().wq_last_device_error().decode()
        super().__init__("%s: %s (status %d)" % (where, text, status))


def lib():
    """Load libwq.so (built in place by weight_only_quantized_dequant_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libwq.so is not built (%s); run `python -m weight_only_quantized_dequant_amd.build`" % LIB_PATH)
        # torch ships its own HIP runtime (file libamdhip64.so, soname libamdhip64.so.7). Loaded
        # first, it also serves libwq.so, whose dependency is that soname; loaded after libwq.so,
        # torch's copy would come in as a second HIP runtime beside the system one, and the
        # launches of one would not run on the device state (memory, current device) of the
        # other. So torch, when present, is loaded before the library.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        L.wq_version.restype = ctypes.c_int
        L.wq_status_string.restype = ctypes.c_char_p
        L.wq_status_string.argtypes = [ctypes.c_int]
        L.wq_last_device_error.restype = ctypes.c_char_p
        L.wq_last_device_error.argtypes = []
        for name in ("wq_packed_bytes", "wq_scales_bytes", "wq_zeros_bytes"):
            f = getattr(L, name)
            f.restype = ctypes.c_size_t
            f.argtypes = [ctypes.c_int, _i64, _i64]
        L.wq_pack_int8.argtypes = [_p, _i64, _i64, _p, _p]
        L.wq_pack_int4.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.wq_pack_fp6.argtypes = [_p, _i64, _i64, _p, _p]
        L.wq_pack_fp4.argtypes = [_p, _i64, _i64, _p, _p]
        L.wq_pack_fp5.argtypes = [_p, _i64, _i64, _p, _p]
        L.wq_unpack.argtypes = [ctypes.c_int, _p, _p, _p, _i64, _i64, _p, _p, _p]
        L.wq_dequant.argtypes = [ctypes.c_int, _p, _p, _p, _p, _i64, _i64, _p]
        L.wq_linear.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, ctypes.c_int, _p]
        L.wq_linear_grouped.argtypes = [ctypes.POINTER(LinearItem), ctypes.c_int, _i64, ctypes.c_int, _p]
        L.wq_linear_grouped.restype = ctypes.c_int
        L.wq_linear_kernel_name.restype = ctypes.c_char_p
        L.wq_linear_kernel_name.argtypes = [ctypes.c_int, _i64, _i64, _i64]
        L.wq_linear_grouped_kernel_name.restype = ctypes.c_char_p
        L.wq_linear_grouped_kernel_name.argtypes = [ctypes.c_int, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.c_int]
        for name in ("wq_pack_int8", "wq_pack_int4", "wq_pack_fp6", "wq_pack_fp4", "wq_pack_fp5", "wq_unpack",
                     "wq_dequant", "wq_linear"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status, where):
    if status != 0:
        raise WqError(status, where)


def _host_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None and a.size else None


def _dev_ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ------------------------------------------------------------------ sizes
def wq_version():
    return lib().wq_version()


def wq_status_string(status):
    return lib().wq_status_string(status).decode()


def wq_last_device_error():
    """Name of the HIP error behind this thread's latest WQ_ERR_DEVICE, or "none"."""
    return lib().wq_last_device_error().decode()


def wq_packed_bytes(fmt, n, k):
    return lib().wq_packed_bytes(fmt, n, k)


def wq_scales_bytes(fmt, n, k):
    return lib().wq_scales_bytes(fmt, n, k)


def wq_zeros_bytes(fmt, n, k):
    return lib().wq_zeros_bytes(fmt, n, k)


def wq_linear_kernel_name(fmt, m, n, k):
    return lib().wq_linear_kernel_name(fmt, m, n, k).decode()


def wq_linear_grouped_kernel_name(fmt, m, shapes):
    ns = (_i64 * len(shapes))(*[n for n, _ in shapes])
    ks = (_i64 * len(shapes))(*[k for _, k in shapes])
    return lib().wq_linear_grouped_kernel_name(fmt, m, ns, ks, len(shapes)).decode()


# ------------------------------------------------------------------ host: pack / unpack
def _w_host(w):
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    return w


def _alloc(fmt, n, k):
    packed = np.empty(max(wq_packed_bytes(fmt, n, k), 1), dtype=np.uint8)
    scales = np.empty(max(wq_scales_bytes(fmt, n, k) // 2, 1), dtype=np.uint16)
    zeros = np.empty(max(wq_zeros_bytes(fmt, n, k) // 2, 1), dtype=np.uint16)
    return packed, scales, zeros


def wq_pack_int8(w):
    """fp32 W [N,K] -> (packed uint8, scales uint16 [N])."""
    w = _w_host(w)
    n, k = w.shape
    packed, scales, _ = _alloc(FMT_W8, n, k)
    _check(lib().wq_pack_int8(_host_ptr(w), n, k, _host_ptr(packed), _host_ptr(scales)), "wq_pack_int8")
    return packed, scales


def wq_pack_int4(w):
    """fp32 W [N,K] -> (packed uint8, scales uint16 [N*K/32], zeros uint16 [N*K/32])."""
    w = _w_host(w)
    n, k = w.shape
    packed, scales, zeros = _alloc(FMT_W4G32, n, k)
    _check(lib().wq_pack_int4(_host_ptr(w), n, k, _host_ptr(packed), _host_ptr(scales), _host_ptr(zeros)), "wq_pack_int4")
    return packed, scales, zeros


def wq_pack_fp6(w):
    """fp32 W [N,K] -> (packed uint8, scales uint16 [N])."""
    w = _w_host(w)
    n, k = w.shape
    packed, scales, _ = _alloc(FMT_W6E3M2, n, k)
    _check(lib().wq_pack_fp6(_host_ptr(w), n, k, _host_ptr(packed), _host_ptr(scales)), "wq_pack_fp6")
    return packed, scales


def wq_pack_fp4(w):
    """fp32 W [N,K] -> (packed uint8, scales uint16 [N])."""
    w = _w_host(w)
    n, k = w.shape
    packed, scales, _ = _alloc(FMT_W4E2M1, n, k)
    _check(lib().wq_pack_fp4(_host_ptr(w), n, k, _host_ptr(packed), _host_ptr(scales)), "wq_pack_fp4")
    return packed, scales


def wq_pack_fp5(w):
    """fp32 W [N,K] -> (packed uint8, scales uint16 [N])."""
    w = _w_host(w)
    n, k = w.shape
    packed, scales, _ = _alloc(FMT_W5E2M2, n, k)
    _check(lib().wq_pack_fp5(_host_ptr(w), n, k, _host_ptr(packed), _host_ptr(scales)), "wq_pack_fp5")
    return packed, scales


def wq_unpack(fmt, packed, scales, zeros, n, k):
    """packed (host) -> (logical codes [N,K], scales copy, zeros copy)."""
    dtype = {FMT_W8: np.int8, FMT_W4G32: np.uint8, FMT_W6E3M2: np.uint8, FMT_W4E2M1: np.uint8,
             FMT_F16: np.uint16, FMT_BF16: np.uint16}.get(fmt, np.uint8)
    codes = np.empty((n, k), dtype=dtype)
    s_out = np.empty(max(wq_scales_bytes(fmt, n, k) // 2, 1), dtype=np.uint16)
    z_out = np.empty(max(wq_zeros_bytes(fmt, n, k) // 2, 1), dtype=np.uint16)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.uint16) if scales is not None else None
    zc = np.ascontiguousarray(zeros, dtype=np.uint16) if zeros is not None else None
    _check(lib().wq_unpack(fmt, _host_ptr(packed), _host_ptr(sc), _host_ptr(zc), n, k, _host_ptr(codes),
                           _host_ptr(s_out), _host_ptr(z_out)), "wq_unpack")
    return codes, s_out, z_out


# ------------------------------------------------------------------ device
def wq_dequant(fmt, packed, scales, zeros, w_out, n, k, stream=None):
    """Device: packed (torch uint8 on the GPU) -> w_out (torch int16/uint16-sized [N,K] on the GPU), async."""
    _check(lib().wq_dequant(fmt, _dev_ptr(packed), _dev_ptr(scales), _dev_ptr(zeros), _dev_ptr(w_out), n, k,
                            _stream_ptr(stream)), "wq_dequant")


def wq_linear(x, packed_w, scales, zeros, y, m, n, k, fmt, stream=None):
    """Device: y[M,N] = x[M,K] . dequant(W)[N,K]^T on torch device buffers, async on stream."""
    _check(lib().wq_linear(_dev_ptr(x), _dev_ptr(packed_w), _dev_ptr(scales), _dev_ptr(zeros), _dev_ptr(y), m, n, k,
                           fmt, _stream_ptr(stream)), "wq_linear")


def wq_linear_grouped(items, m, fmt, stream=None):
    """Device: several independent linears in one launch. items: sequence of
    (x, packed_w, scales, zeros, y, n, k) with torch device buffers; async on stream."""
    arr = (LinearItem * max(1, len(items)))()
    for i, (x, pw, sc, z, y, n, k) in enumerate(items):
        arr[i] = LinearItem(x.data_ptr(), pw.data_ptr(), sc.data_ptr() if sc is not None else None,
                            z.data_ptr() if z is not None else None, y.data_ptr(), n, k)
    _check(lib().wq_linear_grouped(arr, len(items), m, fmt, _stream_ptr(stream)), "wq_linear_grouped")
