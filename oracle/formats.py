"""Number formats: fp16 and bfloat16 rounding, the FP6 e3m2 code, and the FP4 e2m1 and FP5 e2m2 codes.

Test infrastructure only (see the package docstring for who may import it).

FP6 is named, with no bit layout, on the FP6-LLM news page (m.zhengruan.com),
sections "用FP6跑Llama，单卡比双卡还快" and "重新设计内核方案". The reading used here
is e3m2: 1 sign bit, 3 exponent bits with bias 3, 2 mantissa bits, subnormals when the
exponent field is 0, no infinities or NaNs, largest magnitude 28.

The same page says the kernel design serves weights of other bit widths as well, and
names none. FP4 is taken here as e2m1: 1 sign bit, 2 exponent bits with bias 1, 1
mantissa bit, subnormals when the exponent field is 0, no infinities or NaNs, largest
magnitude 6 (the eight magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6). FP5 is taken as e2m2 in the
same family: 1 sign bit, 2 exponent bits with bias 1, 2 mantissa bits, subnormals when the
exponent field is 0, no infinities or NaNs, largest magnitude 7 (the sixteen magnitudes
0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7).

bfloat16 is the activation type named besides fp16 by the gpt-fast guide (www.jsqmd.com,
section "混合精度训练与推理") and the speed-up strategies page (sharktoolz.top, section 4
"Reduce model weight"): the 8-bit exponent of binary32 with 8 significant bits (7 stored),
rounded to nearest with ties to even.
"""

import numpy as np

E3M2_BIAS = 3
E3M2_MAX = 28.0
E2M1_BIAS = 1
E2M1_MAX = 6.0
E2M2_BIAS = 1
E2M2_MAX = 7.0


def fp16_bits(values):
    """Round float64 values to fp16 (round to nearest, ties to even) and return the bit patterns.

    numpy converts float64 to float16 in one correctly rounded step. Values at or
    above 65520 in magnitude become +-inf, as IEEE rounding dictates.
    """
    a = np.asarray(values, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a.astype(np.float16).view(np.uint16)


def fp16_from_bits(bits):
    """fp16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return b.view(np.float16).astype(np.float64)


BF16_MIN_EXP = -126          # smallest normal binade 2^-126; below it the spacing stays 2^-133
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_bits(values):
    """Round float64 values to bfloat16 (round to nearest, ties to even) and return the bit patterns.

    Written from the definition: a finite value in [2^e, 2^(e+1)) lies on a grid of
    spacing 2^(e-7) (8 significant bits), and below 2^-126 on the subnormal grid of
    spacing 2^-133. The value divided by its spacing is rounded to the nearest integer,
    ties to even (an even multiple has an even last stored bit), and scaled back; both
    steps are exact in float64. A result above the largest finite value becomes +-inf.
    The sign of zero is kept. The rounded value is exact in binary32, whose upper 16
    bits are then the bfloat16 pattern.
    """
    a = np.asarray(values, dtype=np.float64)
    _, ex = np.frexp(np.abs(a))                   # |a| = f 2^ex with f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, BF16_MIN_EXP)
    spacing = np.ldexp(1.0, e - 7)
    with np.errstate(invalid="ignore"):
        r = np.rint(a / spacing) * spacing
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, a), r)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits):
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e3m2_value(code):
    """Value of one 6-bit e3m2 code ``s e2 e1 e0 m1 m0`` (closed form, exact in float64)."""
    code = int(code)
    if not 0 <= code < 64:
        raise ValueError("e3m2 code out of range: %r" % code)
    sign = -1.0 if (code >> 5) & 1 else 1.0
    e = (code >> 2) & 7
    m = code & 3
    if e == 0:
        mag = m * 2.0 ** (1 - E3M2_BIAS) / 4.0          # subnormal: 0.m x 2^(1-bias)
    else:
        mag = (1.0 + m / 4.0) * 2.0 ** (e - E3M2_BIAS)  # normal: 1.m x 2^(e-bias)
    return sign * mag


def e3m2_table():
    """All 64 code values as float64 (code 32 is -0.0)."""
    return np.array([e3m2_value(c) for c in range(64)], dtype=np.float64)


def e3m2_encode(t):
    """Encode float64 values as e3m2 codes: nearest magnitude, ties to the even code, saturating.

    The sign bit is the sign bit of ``t`` (so a negative value that rounds to zero gives
    code 32, i.e. -0). The magnitude code is the one among the 32 non-negative values
    nearest to ``|t|``; when two are equally near, the one with an even code wins.
    Magnitudes above 28 are nearest to 28 and so saturate there. This is written as a
    brute-force search over all 32 magnitudes, not as bit manipulation.
    """
    t = np.asarray(t, dtype=np.float64)
    if not np.all(np.isfinite(t)):
        raise ValueError("e3m2_encode: non-finite input")
    mags = e3m2_table()[:32].reshape(1, -1)       # increasing: 0, 1/16, ..., 28
    even = (np.arange(32) % 2 == 0).reshape(1, -1)
    flat = t.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 16
    for i in range(0, flat.size, step):
        # above 28 every magnitude is nearest to 28; clamping first keeps the float64
        # distances below exact (Sterbenz) so that a tie is found only where one exists
        a = np.minimum(np.abs(flat[i:i + step]), E3M2_MAX).reshape(-1, 1)
        dist = np.abs(a - mags)
        is_min = dist == dist.min(axis=1, keepdims=True)
        # at most two codes tie and they are adjacent, so exactly one of them is even
        n_min = is_min.sum(axis=1)
        mag_code = np.where(n_min > 1, np.argmax(is_min & even, axis=1), np.argmax(is_min, axis=1))
        sign = np.signbit(flat[i:i + step]).astype(np.uint8)
        out[i:i + step] = mag_code.astype(np.uint8) | (sign << 5)
    return out.reshape(t.shape)


def e2m1_value(code):
    """Value of one 4-bit e2m1 code ``s e1 e0 m0`` (closed form, exact in float64)."""
    code = int(code)
    if not 0 <= code < 16:
        raise ValueError("e2m1 code out of range: %r" % code)
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = m * 2.0 ** (1 - E2M1_BIAS) / 2.0          # subnormal: 0.m x 2^(1-bias)
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - E2M1_BIAS)  # normal: 1.m x 2^(e-bias)
    return sign * mag


def e2m1_table():
    """All 16 code values as float64 (code 8 is -0.0)."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_encode(t):
    """Encode float64 values as e2m1 codes: nearest magnitude, ties to the even code, saturating.

    As for e3m2: the sign bit is the sign bit of ``t`` (a negative value that rounds to
    zero gives code 8, i.e. -0), the magnitude is the nearest of the 8 non-negative
    values, a tie goes to the even code, and magnitudes above 6 saturate at 6. Written as
    a brute-force search over the 8 magnitudes.
    """
    t = np.asarray(t, dtype=np.float64)
    if not np.all(np.isfinite(t)):
        raise ValueError("e2m1_encode: non-finite input")
    mags = e2m1_table()[:8].reshape(1, -1)        # increasing: 0, 0.5, 1, 1.5, 2, 3, 4, 6
    even = (np.arange(8) % 2 == 0).reshape(1, -1)
    flat = t.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 16
    for i in range(0, flat.size, step):
        a = np.minimum(np.abs(flat[i:i + step]), E2M1_MAX).reshape(-1, 1)
        dist = np.abs(a - mags)
        is_min = dist == dist.min(axis=1, keepdims=True)
        n_min = is_min.sum(axis=1)
        mag_code = np.where(n_min > 1, np.argmax(is_min & even, axis=1), np.argmax(is_min, axis=1))
        sign = np.signbit(flat[i:i + step]).astype(np.uint8)
        out[i:i + step] = mag_code.astype(np.uint8) | (sign << 3)
    return out.reshape(t.shape)


def e2m2_value(code):
    """Value of one 5-bit e2m2 code ``s e1 e0 m1 m0`` (closed form, exact in float64)."""
    code = int(code)
    if not 0 <= code < 32:
        raise ValueError("e2m2 code out of range: %r" % code)
    sign = -1.0 if (code >> 4) & 1 else 1.0
    e = (code >> 2) & 3
    m = code & 3
    if e == 0:
        mag = (m / 4.0) * 2.0 ** (1 - E2M2_BIAS)        # subnormal: 0.m x 2^(1-bias)
    else:
        mag = (1.0 + m / 4.0) * 2.0 ** (e - E2M2_BIAS)  # normal: 1.m x 2^(e-bias)
    return sign * mag


def e2m2_table():
    """All 32 code values as float64 (code 16 is -0.0)."""
    return np.array([e2m2_value(c) for c in range(32)], dtype=np.float64)


def e2m2_encode(t):
    """Encode float64 values as e2m2 codes: nearest magnitude, ties to the even code, saturating.

    As for e2m1: the sign bit is the sign bit of ``t`` (a negative value that rounds to
    zero gives code 16, i.e. -0), the magnitude is the nearest of the 16 non-negative
    values, a tie goes to the even code, and magnitudes above 7 saturate at 7. Written as
    a brute-force search over the 16 magnitudes.
    """
    t = np.asarray(t, dtype=np.float64)
    if not np.all(np.isfinite(t)):
        raise ValueError("e2m2_encode: non-finite input")
    mags = e2m2_table()[:16].reshape(1, -1)       # increasing: 0, 0.25, ..., 6, 7
    even = (np.arange(16) % 2 == 0).reshape(1, -1)
    flat = t.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 15
    for i in range(0, flat.size, step):
        a = np.minimum(np.abs(flat[i:i + step]), E2M2_MAX).reshape(-1, 1)
        dist = np.abs(a - mags)
        is_min = dist == dist.min(axis=1, keepdims=True)
        n_min = is_min.sum(axis=1)
        mag_code = np.where(n_min > 1, np.argmax(is_min & even, axis=1), np.argmax(is_min, axis=1))
        sign = np.signbit(flat[i:i + step]).astype(np.uint8)
        out[i:i + step] = mag_code.astype(np.uint8) | (sign << 4)
    return out.reshape(t.shape)
