"""Quantizers: fp32 weights W[N,K] -> integer codes plus fp16 metadata.

Test infrastructure only (see the package docstring for who may import it).

Pages: the gpt-fast write-up (m.greenbasetech.com) motivates int8 weight quantization,
then int4 with groupwise quantization to recover accuracy. The gpt-fast guide
(www.jsqmd.com), section "量化技术深度解析", gives the int4 group size, 32. The FP6-LLM
news page (m.zhengruan.com) gives FP6 weights with fp16 activations (W6A16).

The pages give no formulas. The readings are:

* int8: symmetric, one fp16 scale per output row, ``s = fp16(max|w| / 127)``,
  ``q = clamp(rint(w / s), -127, 127)``.
* int4: asymmetric, groups of 32 consecutive K within a row. ``lo = min(min w, 0)``,
  ``hi = max(max w, 0)``, ``s = fp16((hi - lo) / 15)``, ``z = clamp(rint(-lo / s), 0, 15)``,
  ``q = clamp(rint(w / s) + z, 0, 15)``. The zero point z is an integer stored as fp16,
  and the dequantised weight is ``(q - z) * s``.
* int3 (a further bit width through the same design, as the FP6-LLM news page
  (m.zhengruan.com), section "重新设计内核方案", has one kernel design serve several bit
  widths; the page names no 3-bit format): int4's rule with 7 in place of 15, i.e.
  ``s = fp16((hi - lo) / 7)``, ``z = clamp(rint(-lo / s), 0, 7)``, ``q = clamp(rint(w / s) + z, 0, 7)``.
* FP6: one fp16 scale per output row, ``s = fp16(max|w| / 28)``, code = e3m2 encoding of
  ``w / s`` (nearest, ties to even code, saturating at 28).
* FP4 (a further bit width through the same design; the page names none): e2m1 with one
  fp16 scale per output row, ``s = fp16(max|w| / 6)``, code = e2m1 encoding of ``w / s``.
* FP5 (the same): e2m2 with one fp16 scale per output row, ``s = fp16(max|w| / 7)``, code =
  e2m2 encoding of ``w / s``.
* In all of them a scale that rounds to 0 makes every code of its row (or group) 0, and
  z = 0. A scale that overflows fp16 is an error.

Arithmetic: each quotient is one IEEE float64 operation on float64 copies of the fp32
weights and of the fp16 scale, then one rounding (``rint`` ties to even, or fp16 RNE).
"""

import numpy as np

from .formats import fp16_bits, fp16_from_bits, e3m2_encode, e2m1_encode, e2m2_encode, E2M1_MAX, E2M2_MAX


class OracleRangeError(ValueError):
    """A weight is non-finite, or a scale would not fit in fp16."""


def _check_w(w):
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise TypeError("weights must be a 2-D float32 array")
    if not np.all(np.isfinite(w)):
        raise OracleRangeError("non-finite weight")
    return w.astype(np.float64)


def _scale16(x):
    bits = fp16_bits(x)
    if np.any(np.isinf(fp16_from_bits(bits))):
        raise OracleRangeError("scale overflows fp16")
    return bits


def quantize_int8(w):
    """int8 per output row. Returns (q int8 [N,K], scale bits uint16 [N])."""
    w = _check_w(w)
    amax = np.max(np.abs(w), axis=1)
    s_bits = _scale16(amax / 127.0)
    s = fp16_from_bits(s_bits)
    q = np.zeros(w.shape, dtype=np.int8)
    nz = s > 0
    q[nz] = np.clip(np.rint(w[nz] / s[nz, None]), -127, 127).astype(np.int8)
    return q, s_bits


def quantize_int4_g32(w):
    """int4 asymmetric, group 32 along K. Returns (q uint8 [N,K] in 0..15, scale bits [N,K/32], zero bits [N,K/32])."""
    return _asymmetric_g32(w, 15)


def quantize_int3_g32(w):
    """int3 asymmetric, group 32 along K. Returns (q uint8 [N,K] in 0..7, scale bits [N,K/32], zero bits [N,K/32])."""
    return _asymmetric_g32(w, 7)


def _asymmetric_g32(w, top):
    """Codes 0..top with an fp16 scale and an integer zero point per group of 32 consecutive K."""
    w = _check_w(w)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    g = w.reshape(n, k // 32, 32)
    lo = np.minimum(g.min(axis=2), 0.0)
    hi = np.maximum(g.max(axis=2), 0.0)
    s_bits = _scale16((hi - lo) / float(top))
    s = fp16_from_bits(s_bits)
    q = np.zeros(g.shape, dtype=np.uint8)
    z = np.zeros(s.shape, dtype=np.float64)
    nz = s > 0
    # + 0.0 turns the -0 that rint(-0/s) yields for a group with lo = 0 into the integer 0
    z[nz] = np.clip(np.rint(-lo[nz] / s[nz]), 0, top) + 0.0
    q[nz] = np.clip(np.rint(g[nz] / s[nz][:, None]) + z[nz][:, None], 0, top).astype(np.uint8)
    return q.reshape(n, k), s_bits, fp16_bits(z)


def quantize_fp6(w):
    """FP6 e3m2 per output row. Returns (codes uint8 [N,K] in 0..63, scale bits uint16 [N])."""
    w = _check_w(w)
    amax = np.max(np.abs(w), axis=1)
    s_bits = _scale16(amax / 28.0)
    s = fp16_from_bits(s_bits)
    codes = np.zeros(w.shape, dtype=np.uint8)
    nz = s > 0
    if np.any(nz):
        codes[nz] = e3m2_encode(w[nz] / s[nz, None])
    return codes, s_bits


def quantize_fp4(w):
    """FP4 e2m1 per output row. Returns (codes uint8 [N,K] in 0..15, scale bits uint16 [N])."""
    w = _check_w(w)
    amax = np.max(np.abs(w), axis=1)
    s_bits = _scale16(amax / E2M1_MAX)
    s = fp16_from_bits(s_bits)
    codes = np.zeros(w.shape, dtype=np.uint8)
    nz = s > 0
    if np.any(nz):
        codes[nz] = e2m1_encode(w[nz] / s[nz, None])
    return codes, s_bits


def quantize_fp5(w):
    """FP5 e2m2 per output row. Returns (codes uint8 [N,K] in 0..31, scale bits uint16 [N])."""
    w = _check_w(w)
    amax = np.max(np.abs(w), axis=1)
    s_bits = _scale16(amax / E2M2_MAX)
    s = fp16_from_bits(s_bits)
    codes = np.zeros(w.shape, dtype=np.uint8)
    nz = s > 0
    if np.any(nz):
        codes[nz] = e2m2_encode(w[nz] / s[nz, None])
    return codes, s_bits
