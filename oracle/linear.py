"""Dequantisation to fp16 or bfloat16 and the reference linear layer.

Test infrastructure only (see the package docstring for who may import it).

The FP6-LLM news page (m.zhengruan.com), section "重新设计内核方案", describes the
computation: the low-bit weights are turned back into fp16 values and the layer is then
an fp16 matrix product, ``y = x . W^T``. The pages do not state a precision for the
product. The reading used here is fp32 accumulation with fp16 inputs and outputs. The
reference below is therefore the exact sum, computed in float64, of the fp16 inputs
times the fp16 dequantised weights. A device result is accepted when it lies within the
bound given by ``error_bound``.

With bfloat16 activations (named besides fp16 by the gpt-fast guide, www.jsqmd.com,
section "混合精度训练与推理", and by the speed-up strategies page, sharktoolz.top,
section 4 "Reduce model weight") the same statement holds with bfloat16 in place of
fp16: x, the dequantised weights and y are bfloat16, the sum is fp32.
"""

import numpy as np

from .formats import fp16_bits, fp16_from_bits, bf16_bits, bf16_from_bits, e3m2_table, e2m1_table, e2m2_table
from .layout import (FMT_F16, FMT_W8, FMT_W4G32, FMT_W6E3M2, FMT_W4E2M1, FMT_BF16, FMT_W5E2M2, FMT_W3G32,
                     FMT_W6E3M2_P24, pack_vectorized)

# activation types: how x, the dequantised weights and y are stored
ACT_F16 = "f16"
ACT_BF16 = "bf16"
_ROUND = {ACT_F16: fp16_bits, ACT_BF16: bf16_bits}
_VALUE = {ACT_F16: fp16_from_bits, ACT_BF16: bf16_from_bits}
_UNIT_ROUNDOFF = {ACT_F16: 2.0 ** -11, ACT_BF16: 2.0 ** -8}
from .quantize import quantize_int8, quantize_int4_g32, quantize_fp6, quantize_fp4, quantize_fp5, quantize_int3_g32


def dequant_values(fmt, codes, scales=None, zeros=None):
    """Logical codes + fp16 metadata bits -> the exact dequantised values as float64 [N,K].

    W8: q * s. W4 and W3: (q - z) * s with s, z of the weight's group. W6 and P24 (the same
    codes in another layout): e3m2(c) * s. FP4: e2m1(c) * s. FP5: e2m2(c) * s. Each product is exact in float64 (the factors have at
    most 11 and 8 significant bits). Not defined for the unquantized formats.
    """
    codes = np.asarray(codes)
    n, k = codes.shape
    s = fp16_from_bits(scales)
    if fmt == FMT_W8:
        v = codes.astype(np.float64) * s.reshape(n, 1)
    elif fmt in (FMT_W4G32, FMT_W3G32):
        z = fp16_from_bits(zeros).reshape(n, k // 32, 1)
        q = codes.astype(np.float64).reshape(n, k // 32, 32)
        v = ((q - z) * s.reshape(n, k // 32, 1)).reshape(n, k)
    elif fmt in (FMT_W6E3M2, FMT_W6E3M2_P24):
        v = e3m2_table()[codes.astype(np.int64)] * s.reshape(n, 1)
    elif fmt == FMT_W4E2M1:
        v = e2m1_table()[codes.astype(np.int64)] * s.reshape(n, 1)
    elif fmt == FMT_W5E2M2:
        v = e2m2_table()[codes.astype(np.int64)] * s.reshape(n, 1)
    else:
        raise ValueError("unknown format %r" % fmt)
    return v


def dequant_fp16(fmt, codes, scales=None, zeros=None):
    """Logical codes + fp16 metadata bits -> dequantised weights as fp16 bits [N,K]:
    the exact value of ``dequant_values`` rounded once to fp16. F16: the weights themselves."""
    if fmt == FMT_F16:
        return np.asarray(codes).astype(np.uint16)
    return fp16_bits(dequant_values(fmt, codes, scales, zeros))


def dequant_bf16(fmt, codes, scales=None, zeros=None):
    """The same, rounded once to bfloat16. BF16: the weights themselves."""
    if fmt == FMT_BF16:
        return np.asarray(codes).astype(np.uint16)
    return bf16_bits(dequant_values(fmt, codes, scales, zeros))


def linear_ref(x_bits, w_bits, act=ACT_F16):
    """y[m,n] = sum_k x[m,k] * w[n,k] in float64, for fp16 (or bfloat16) bit inputs x [M,K] and w [N,K]."""
    x = _VALUE[act](x_bits)
    w = _VALUE[act](w_bits)
    return x @ w.T


def error_bound(x_bits, w_bits, y_ref, act=ACT_F16):
    """Largest error allowed for a device output, element by element.

    With inputs of unit roundoff u (2^-11 for fp16, 2^-8 for bfloat16), fp32
    accumulation over K terms and one final rounding to the same type, a result is
    accepted when
        |y - y_ref| <= u |y_ref| + (u + K 2^-23) S + 2^-25 A + 2^-24
    where S = sum_k |x w| and A = sum_k |x|. The terms cover: the output rounding; a
    per-row or per-group scale applied after the sum instead of to every weight; the
    fp32 summation in any order; fp16 subnormal weights; a subnormal output.
    """
    x = np.abs(_VALUE[act](x_bits))
    w = np.abs(_VALUE[act](w_bits))
    u = _UNIT_ROUNDOFF[act]
    k = x.shape[1]
    s = x @ w.T
    a = x.sum(axis=1, keepdims=True)
    return u * np.abs(y_ref) + (u + k * 2.0 ** -23) * s + 2.0 ** -25 * a + 2.0 ** -24


def quantize_and_pack(fmt, w):
    """fp32 W [N,K] -> (packed bytes, scale bits, zero bits, logical codes), all as numpy arrays."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if fmt == FMT_W8:
        codes, s = quantize_int8(w)
        z = np.zeros(0, dtype=np.uint16)
    elif fmt == FMT_W4G32:
        codes, s, z = quantize_int4_g32(w)
    elif fmt == FMT_W3G32:
        codes, s, z = quantize_int3_g32(w)
    elif fmt in (FMT_W6E3M2, FMT_W6E3M2_P24):
        codes, s = quantize_fp6(w)
        z = np.zeros(0, dtype=np.uint16)
    elif fmt == FMT_W4E2M1:
        codes, s = quantize_fp4(w)
        z = np.zeros(0, dtype=np.uint16)
    elif fmt == FMT_W5E2M2:
        codes, s = quantize_fp5(w)
        z = np.zeros(0, dtype=np.uint16)
    elif fmt in (FMT_F16, FMT_BF16):
        codes = _ROUND[ACT_F16 if fmt == FMT_F16 else ACT_BF16](w.astype(np.float64))
        s = np.zeros(0, dtype=np.uint16)
        z = np.zeros(0, dtype=np.uint16)
    else:
        raise ValueError("unknown format %r" % fmt)
    return pack_vectorized(fmt, codes), s, z, codes
