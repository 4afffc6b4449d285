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
FMT_W3G32, FMT_W6E3M2_P24 = 7, 8
FMT_NAMES = {"f16": FMT_F16, "w8": FMT_W8, "w4g32": FMT_W4G32, "w6e3m2": FMT_W6E3M2, "w4e2m1": FMT_W4E2M1,
             "bf16": FMT_BF16, "w5e2m2": FMT_W5E2M2, "w3g32": FMT_W3G32, "w6e3m2_p24": FMT_W6E3M2_P24}
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
        L.wq_pack_int3.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.wq_pack_fp6_p24.argtypes = [_p, _i64, _i64, _p, _p]
        L.wq_unpack.argtypes = [ctypes.c_int, _p, _p, _p, _i64, _i64, _p, _p, _p]
        L.wq_dequant.argtypes = [ctypes.c_int, _p, _p, _p, _p, _i64, _i64, _p]
        L.wq_linear.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, ctypes.c_int, _p]
        L.wq_linear_grouped.argtypes = [ctypes.POINTER(LinearItem), ctypes.c_int, _i64, ctypes.c_int, _p]
        L.wq_linear_silu.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, ctypes.c_int, _p]
        L.wq_linear_silu.restype = ctypes.c_int
        L.wq_linear_grouped.restype = ctypes.c_int
        L.wq_linear_kernel_name.restype = ctypes.c_char_p
        L.wq_linear_kernel_name.argtypes = [ctypes.c_int, _i64, _i64, _i64]
        L.wq_linear_grouped_kernel_name.restype = ctypes.c_char_p
        L.wq_linear_grouped_kernel_name.argtypes = [ctypes.c_int, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.c_int]
        for name in ("wq_pack_int8", "wq_pack_int4", "wq_pack_fp6", "wq_pack_fp4", "wq_pack_fp5", "wq_pack_int3",
                     "wq_pack_fp6_p24", "wq_unpack",
                     "wq_dequant", "wq_linear"):
            getattr(L, name).restype = ctypes.c_int
        # decode-step calls (include/wq_decode.h)
        L.wq_rope_table.argtypes = [ctypes.c_double, _i64, _i64, _p, _p]
        L.wq_embed.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p]
        L.wq_add_rmsnorm.argtypes = [_p, _p, _p, ctypes.c_float, _p, _i64, _i64, _p]
        L.wq_attention_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
        L.wq_attention_workspace_bytes.restype = ctypes.c_size_t
        L.wq_rope_attention.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p,
                                        ctypes.c_size_t, _p]
        L.wq_rope_attention_noalloc.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p]
        L.wq_rope_attention_noalloc.restype = ctypes.c_int
        L.wq_silu_mul.argtypes = [_p, _p, _p, _i64, _p]
        L.wq_argmax_next.argtypes = [_p, _i64, _i64, _p, _p, _p]
        for name in ("wq_rope_table", "wq_embed", "wq_add_rmsnorm", "wq_rope_attention", "wq_silu_mul", "wq_argmax_next"):
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


def wq_pack_int3(w):
    """fp32 W [N,K] -> (packed uint8, scales uint16 [N*K/32], zeros uint16 [N*K/32])."""
    w = _w_host(w)
    n, k = w.shape
    packed, scales, zeros = _alloc(FMT_W3G32, n, k)
    _check(lib().wq_pack_int3(_host_ptr(w), n, k, _host_ptr(packed), _host_ptr(scales), _host_ptr(zeros)), "wq_pack_int3")
    return packed, scales, zeros


def wq_pack_fp6_p24(w):
    """fp32 W [N,K] -> (packed uint8 in the 2+4 split layout, scales uint16 [N])."""
    w = _w_host(w)
    n, k = w.shape
    packed, scales, _ = _alloc(FMT_W6E3M2_P24, n, k)
    _check(lib().wq_pack_fp6_p24(_host_ptr(w), n, k, _host_ptr(packed), _host_ptr(scales)), "wq_pack_fp6_p24")
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
# The C ABI sees raw pointers and can check only their alignment. Before a device call the
# binding checks every buffer the kernels will touch: a GPU tensor on the current device,
# contiguous, and at least as many bytes as (fmt, M, N, K) imply. A CPU tensor, a strided view
# or a short buffer would otherwise become out-of-bounds device accesses.
def _valid_shape(m, n, k):
    return m >= 1 and n >= 1 and k >= 32 and k % 32 == 0


def _need(t, nbytes, name, where):
    if t is None:
        return          # a missing required buffer is the library's WQ_ERR_ARG
    if not getattr(t, "is_cuda", False):
        raise ValueError("%s: %s must be a GPU tensor" % (where, name))
    import torch
    if t.get_device() != torch.cuda.current_device():
        raise ValueError("%s: %s is on device %d, not the current device %d" % (where, name, t.get_device(),
                                                                                  torch.cuda.current_device()))
    if not t.is_contiguous():
        raise ValueError("%s: %s must be contiguous" % (where, name))
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s: %s holds %d bytes; the call reads or writes %d" % (where, name, have, nbytes))


def _check_linear_buffers(x, packed_w, scales, zeros, y, m, n, k, fmt, where, y_rows=None):
    """y_rows: the output's columns when they are not n (wq_linear_silu writes n / 2)."""
    sized = _valid_shape(m, n, k) and wq_packed_bytes(fmt, n, k) > 0
    size = (lambda v: v) if sized else (lambda v: 0)
    _need(x, size(2 * m * k), "x", where)
    _need(y, size(2 * m * (n if y_rows is None else y_rows)), "y", where)
    _need(packed_w, size(wq_packed_bytes(fmt, n, k)), "packed_w", where)
    _need(scales, size(wq_scales_bytes(fmt, n, k)), "scales", where)
    _need(zeros, size(wq_zeros_bytes(fmt, n, k)), "zeros", where)


def wq_dequant(fmt, packed, scales, zeros, w_out, n, k, stream=None):
    """Device: packed (torch uint8 on the GPU) -> w_out (torch int16/uint16-sized [N,K] on the GPU), async."""
    sized = _valid_shape(1, n, k) and wq_packed_bytes(fmt, n, k) > 0
    _need(packed, wq_packed_bytes(fmt, n, k) if sized else 0, "packed", "wq_dequant")
    _need(scales, wq_scales_bytes(fmt, n, k) if sized else 0, "scales", "wq_dequant")
    _need(zeros, wq_zeros_bytes(fmt, n, k) if sized else 0, "zeros", "wq_dequant")
    _need(w_out, 2 * n * k if sized else 0, "w_out", "wq_dequant")
    _check(lib().wq_dequant(fmt, _dev_ptr(packed), _dev_ptr(scales), _dev_ptr(zeros), _dev_ptr(w_out), n, k,
                            _stream_ptr(stream)), "wq_dequant")


def wq_linear(x, packed_w, scales, zeros, y, m, n, k, fmt, stream=None):
    """Device: y[M,N] = x[M,K] . dequant(W)[N,K]^T on torch device buffers, async on stream."""
    _check_linear_buffers(x, packed_w, scales, zeros, y, m, n, k, fmt, "wq_linear")
    _check(lib().wq_linear(_dev_ptr(x), _dev_ptr(packed_w), _dev_ptr(scales), _dev_ptr(zeros), _dev_ptr(y), m, n, k,
                           fmt, _stream_ptr(stream)), "wq_linear")


def wq_linear_silu(x, packed_w, scales, zeros, act, m, f, k, fmt, stream=None):
    """Device: act[M,F] = silu(gate) * up from one packed [2F, K] matrix of gate/up row pairs."""
    _check_linear_buffers(x, packed_w, scales, zeros, act, m, 2 * f, k, fmt, "wq_linear_silu", y_rows=f)
    _check(lib().wq_linear_silu(_dev_ptr(x), _dev_ptr(packed_w), _dev_ptr(scales), _dev_ptr(zeros), _dev_ptr(act), m,
                                f, k, fmt, _stream_ptr(stream)), "wq_linear_silu")


def wq_linear_grouped(items, m, fmt, stream=None):
    """Device: several independent linears in one launch. items: sequence of
    (x, packed_w, scales, zeros, y, n, k) with torch device buffers; async on stream."""
    arr = (LinearItem * max(1, len(items)))()
    for i, (x, pw, sc, z, y, n, k) in enumerate(items):
        _check_linear_buffers(x, pw, sc, z, y, m, n, k, fmt, "wq_linear_grouped item %d" % i)
        arr[i] = LinearItem(x.data_ptr(), pw.data_ptr(), sc.data_ptr() if sc is not None else None,
                            z.data_ptr() if z is not None else None, y.data_ptr(), n, k)
    _check(lib().wq_linear_grouped(arr, len(items), m, fmt, _stream_ptr(stream)), "wq_linear_grouped")


# ------------------------------------------------------------------ decode-step calls (include/wq_decode.h)
def wq_rope_table(theta, head_dim, positions):
    """Host: (cos, sin) float32 [positions, head_dim/2] of the rotary embedding."""
    cos = np.empty((max(positions, 1), max(head_dim // 2, 1)), dtype=np.float32)
    sin = np.empty_like(cos)
    _check(lib().wq_rope_table(theta, head_dim, positions, _host_ptr(cos), _host_ptr(sin)), "wq_rope_table")
    return cos, sin


def wq_embed(table, tokens, x, m, d, vocab, stream=None):
    """Device: x[m] = table[tokens[m]] (fp16 table [vocab, d] -> float32 x [M, d])."""
    sized = m >= 1 and d >= 1 and vocab >= 1
    _need(table, 2 * vocab * d if sized else 0, "table", "wq_embed")
    _need(tokens, 4 * m if sized else 0, "tokens", "wq_embed")
    _need(x, 4 * m * d if sized else 0, "x", "wq_embed")
    _check(lib().wq_embed(_dev_ptr(table), _dev_ptr(tokens), _dev_ptr(x), m, d, vocab, _stream_ptr(stream)), "wq_embed")


def wq_add_rmsnorm(x, delta, g, eps, out, m, d, stream=None):
    """Device: x += delta (if given); out = fp16(rmsnorm(x) * g)."""
    sized = m >= 1 and d >= 1
    _need(x, 4 * m * d if sized else 0, "x", "wq_add_rmsnorm")
    _need(delta, 2 * m * d if sized else 0, "delta", "wq_add_rmsnorm")
    _need(g, 2 * d if sized else 0, "g", "wq_add_rmsnorm")
    _need(out, 2 * m * d if sized else 0, "out", "wq_add_rmsnorm")
    _check(lib().wq_add_rmsnorm(_dev_ptr(x), _dev_ptr(delta), _dev_ptr(g), eps, _dev_ptr(out), m, d, _stream_ptr(stream)),
           "wq_add_rmsnorm")


def wq_attention_workspace_bytes(m, n_heads, head_dim, max_seq):
    return lib().wq_attention_workspace_bytes(m, n_heads, head_dim, max_seq)


def wq_rope_attention(q, k, v, cache_k, cache_v, rope_cos, rope_sin, pos, out, m, n_heads, n_kv_heads, head_dim, max_seq,
                      workspace, stream=None):
    """Device: rotary embedding, key/value cache append and attention of one new token per sequence."""
    where = "wq_rope_attention"
    sized = min(m, n_heads, n_kv_heads, head_dim, max_seq) >= 1
    z = (lambda b: b) if sized else (lambda b: 0)
    _need(q, z(2 * m * n_heads * head_dim), "q", where)
    _need(out, z(2 * m * n_heads * head_dim), "out", where)
    _need(k, z(2 * m * n_kv_heads * head_dim), "k", where)
    _need(v, z(2 * m * n_kv_heads * head_dim), "v", where)
    _need(cache_k, z(2 * m * max_seq * n_kv_heads * head_dim), "cache_k", where)
    _need(cache_v, z(2 * m * max_seq * n_kv_heads * head_dim), "cache_v", where)
    _need(rope_cos, z(4 * max_seq * (head_dim // 2)), "rope_cos", where)
    _need(rope_sin, z(4 * max_seq * (head_dim // 2)), "rope_sin", where)
    _need(pos, z(4), "pos", where)
    ws = wq_attention_workspace_bytes(m, n_heads, head_dim, max_seq) if sized else 0
    _need(workspace, ws, "workspace", where)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wq_rope_attention(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(cache_k), _dev_ptr(cache_v),
                                   _dev_ptr(rope_cos), _dev_ptr(rope_sin), _dev_ptr(pos), _dev_ptr(out), m, n_heads,
                                   n_kv_heads, head_dim, max_seq, _dev_ptr(workspace), have, _stream_ptr(stream)), where)


def wq_silu_mul(gate, up, out, n, stream=None):
    """Device: out = fp16(silu(gate) * up), n elements."""
    _need(gate, 2 * max(n, 0), "gate", "wq_silu_mul")
    _need(up, 2 * max(n, 0), "up", "wq_silu_mul")
    _need(out, 2 * max(n, 0), "out", "wq_silu_mul")
    _check(lib().wq_silu_mul(_dev_ptr(gate), _dev_ptr(up), _dev_ptr(out), n, _stream_ptr(stream)), "wq_silu_mul")


def wq_argmax_next(logits, m, vocab, tokens, pos, stream=None):
    """Device: tokens[m] = argmax(logits[m]) (lowest index of the largest); pos += 1."""
    sized = m >= 1 and vocab >= 1
    _need(logits, 2 * m * vocab if sized else 0, "logits", "wq_argmax_next")
    _need(tokens, 4 * m if sized else 0, "tokens", "wq_argmax_next")
    _need(pos, 4 if sized else 0, "pos", "wq_argmax_next")
    _check(lib().wq_argmax_next(_dev_ptr(logits), m, vocab, _dev_ptr(tokens), _dev_ptr(pos), _stream_ptr(stream)),
           "wq_argmax_next")


NOALLOC_SCRATCH_BYTES = 8 << 20   # WQ_NOALLOC_SCRATCH_BYTES of include/wq_decode.h


def wq_rope_attention_noalloc(q, k, v, cache_k, cache_v, rope_cos, rope_sin, pos, out, m, n_heads, n_kv_heads, head_dim,
                              max_seq, stream=None):
    """Device: wq_rope_attention with its workspace in the library's own per-GPU buffer (no allocation)."""
    where = "wq_rope_attention_noalloc"
    sized = min(m, n_heads, n_kv_heads, head_dim, max_seq) >= 1
    z = (lambda b: b) if sized else (lambda b: 0)
    _need(q, z(2 * m * n_heads * head_dim), "q", where)
    _need(out, z(2 * m * n_heads * head_dim), "out", where)
    _need(k, z(2 * m * n_kv_heads * head_dim), "k", where)
    _need(v, z(2 * m * n_kv_heads * head_dim), "v", where)
    _need(cache_k, z(2 * m * max_seq * n_kv_heads * head_dim), "cache_k", where)
    _need(cache_v, z(2 * m * max_seq * n_kv_heads * head_dim), "cache_v", where)
    _need(rope_cos, z(4 * max_seq * (head_dim // 2)), "rope_cos", where)
    _need(rope_sin, z(4 * max_seq * (head_dim // 2)), "rope_sin", where)
    _need(pos, z(4), "pos", where)
    _check(lib().wq_rope_attention_noalloc(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(cache_k), _dev_ptr(cache_v),
                                           _dev_ptr(rope_cos), _dev_ptr(rope_sin), _dev_ptr(pos), _dev_ptr(out), m,
                                           n_heads, n_kv_heads, head_dim, max_seq, _stream_ptr(stream)), where)
