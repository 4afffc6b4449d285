"""Independent checks that pin the CPU oracle to something other than itself.

Nothing here calls the oracle's own arithmetic. These are exact-rational (Fraction)
statements of the definitions, brute-force searches over every code, and fixtures
typed by hand under tests/golden/. Each ``check_*`` takes the function under test as
an argument, so the same predicate both accepts the oracle and rejects planted
mistakes (see test_oracle_mutations.py).
"""

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- exact rounding
def rint_even(fr):
    """Nearest integer to a Fraction, ties to even."""
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def fp16_round(fr):
    """Round a Fraction to the nearest fp16 value (ties to even). Returns a Fraction, or +-inf as float."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2^e <= a < 2^(e+1) exactly
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                                  # below 2^-14 the spacing stays 2^-24
    quantum = Fraction(2) ** (e - 10)
    n = rint_even(a / quantum)
    v = n * quantum
    if v >= 65536 or (v == 65536):
        return sign * math.inf
    if v > 65504:                                    # rounds past the largest finite value
        return sign * math.inf
    return sign * v


def bf16_round(fr):
    """Round a Fraction to the nearest bfloat16 value (ties to even). Returns a Fraction, or +-inf as float.

    bfloat16: 8 significant bits; normal binades from 2^-126 up, below that the spacing
    stays 2^-133; the largest finite value is (2 - 2^-7) 2^127.
    """
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    v = rint_even(a / quantum) * quantum
    if v > (2 - Fraction(1, 128)) * Fraction(2) ** 127:
        return sign * math.inf
    return sign * v


def check_bf16_rounding(round_fn, values):
    """round_fn(float64 array) -> bfloat16 bits must be the exact round-to-nearest-even of every value."""
    got = round_fn(np.array(values, dtype=np.float64))
    for v, g in zip(values, got):
        r = bf16_round(Fraction(v))
        want = (0x8000 if math.copysign(1.0, v) < 0 else 0) if r == 0 else fraction_to_bf16_bits(r)
        if int(g) != want:
            return False
    return True


def bf16_bits_to_fraction(b):
    """Exact value of a bfloat16 bit pattern from its fields: sign, 8 exponent bits (bias 127), 7 mantissa bits."""
    b = int(b)
    s = -1 if b >> 15 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0xFF:
        raise ValueError("inf/nan")
    if e == 0:
        return s * Fraction(m) * Fraction(2) ** -133
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def fraction_to_bf16_bits(v):
    """Exact bfloat16 value (Fraction, or inf) -> bit pattern, built from the fields; v must be representable."""
    if isinstance(v, float) and math.isinf(v):
        return 0x7F80 if v > 0 else 0xFF80
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(Fraction(v))
    if a < Fraction(2) ** -126:
        m = a / Fraction(2) ** -133
        assert m.denominator == 1
        return sign | int(m)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    m = (a / Fraction(2) ** e - 1) * 128
    assert m.denominator == 1 and 0 <= m < 128
    return sign | ((e + 127) << 7) | int(m)


def f16_bits_to_fraction(b):
    b = int(b)
    s = -1 if b >> 15 else 1
    e = (b >> 10) & 31
    m = b & 1023
    if e == 0:
        return s * Fraction(m, 1 << 24)
    assert e != 31
    return s * Fraction(1024 + m, 1 << 10) * Fraction(2) ** (e - 15)


def fraction_to_f16_bits(v):
    """Exact fp16 value (Fraction, or inf) -> bit pattern; v must be representable."""
    if isinstance(v, float) and math.isinf(v):
        return 0x7C00 if v > 0 else 0xFC00
    return int(np.float16(float(v)).view(np.uint16))  # float(v) is exact for fp16 values


# ---------------------------------------------------------------- e3m2 from the golden table
def golden_e3m2():
    """64 magnitudes as Fractions with the sign of each code: (value, negative?)."""
    rows = []
    with open(os.path.join(GOLDEN, "e3m2_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([Fraction(t) for t in line.split()])
    assert len(rows) == 8 and all(len(r) == 4 for r in rows)
    mags = [rows[c >> 2][c & 3] for c in range(32)]
    return [(mags[c & 31], bool(c & 32)) for c in range(64)]


def check_e3m2_table(value_fn):
    """value_fn(code) must equal the hand-typed table, with -0 for code 32."""
    for c, (mag, neg) in enumerate(golden_e3m2()):
        v = value_fn(c)
        if Fraction(v) != (-mag if neg else mag):
            return False
        if math.copysign(1.0, v) != (-1.0 if neg else 1.0):
            return False
    return True


def golden_e2m1():
    """16 e2m1 magnitudes as Fractions with the sign of each code: (value, negative?)."""
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([Fraction(t) for t in line.split()])
    assert len(rows) == 4 and all(len(r) == 2 for r in rows)
    mags = [rows[c >> 1][c & 1] for c in range(8)]
    return [(mags[c & 7], bool(c & 8)) for c in range(16)]


def check_e2m1_table(value_fn):
    """value_fn(code) must equal the hand-typed e2m1 table, with -0 for code 8."""
    for c, (mag, neg) in enumerate(golden_e2m1()):
        v = value_fn(c)
        if Fraction(v) != (-mag if neg else mag):
            return False
        if math.copysign(1.0, v) != (-1.0 if neg else 1.0):
            return False
    return True


def golden_e2m2():
    """32 e2m2 magnitudes as Fractions with the sign of each code: (value, negative?)."""
    rows = []
    with open(os.path.join(GOLDEN, "e2m2_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([Fraction(t) for t in line.split()])
    assert len(rows) == 4 and all(len(r) == 4 for r in rows)
    mags = [rows[c >> 2][c & 3] for c in range(16)]
    return [(mags[c & 15], bool(c & 16)) for c in range(32)]


def check_e2m2_table(value_fn):
    """value_fn(code) must equal the hand-typed e2m2 table, with -0 for code 16."""
    for c, (mag, neg) in enumerate(golden_e2m2()):
        v = value_fn(c)
        if Fraction(v) != (-mag if neg else mag):
            return False
        if math.copysign(1.0, v) != (-1.0 if neg else 1.0):
            return False
    return True


# ---------------------------------------------------------------- brute-force quantizers
def brute_fp4_code(t):
    """Nearest e2m1 code to a float t: sign from t's sign bit, nearest magnitude, ties to even code."""
    tab = golden_e2m1()
    neg = math.copysign(1.0, t) < 0
    ft = abs(Fraction(t))
    best = None
    for c in range(8):
        d = abs(ft - tab[c][0])
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (8 if neg else 0)


def brute_fp4_row(w_row):
    """(codes, scale bits) for one fp32 row: exact quotient w/s, nearest e2m1 magnitude, ties to even code."""
    amax = max(abs(Fraction(float(v))) for v in w_row)
    s = fp16_round(amax / 6)
    if s == 0:
        return [0] * len(w_row), 0
    tab = golden_e2m1()
    codes = []
    for v in w_row:
        a = abs(Fraction(float(v))) / s
        best = None
        for c in range(8):
            d = abs(a - tab[c][0])
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        codes.append(best[1] | (8 if math.copysign(1.0, float(v)) < 0 else 0))
    return codes, fraction_to_f16_bits(s)


def brute_fp5_code(t):
    """Nearest e2m2 code to a float t: sign from t's sign bit, nearest magnitude, ties to even code."""
    tab = golden_e2m2()
    neg = math.copysign(1.0, t) < 0
    ft = abs(Fraction(t))
    best = None
    for c in range(16):
        d = abs(ft - tab[c][0])
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (16 if neg else 0)


def brute_fp5_row(w_row):
    """(codes, scale bits) for one fp32 row: exact quotient w/s, nearest e2m2 magnitude, ties to even code."""
    amax = max(abs(Fraction(float(v))) for v in w_row)
    s = fp16_round(amax / 7)
    if s == 0:
        return [0] * len(w_row), 0
    tab = golden_e2m2()
    codes = []
    for v in w_row:
        a = abs(Fraction(float(v))) / s
        best = None
        for c in range(16):
            d = abs(a - tab[c][0])
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        codes.append(best[1] | (16 if math.copysign(1.0, float(v)) < 0 else 0))
    return codes, fraction_to_f16_bits(s)


def brute_fp6_code(t):
    """Nearest e3m2 code to a float t: sign from t's sign bit, nearest magnitude, ties to even code."""
    tab = golden_e3m2()
    neg = math.copysign(1.0, t) < 0
    ft = abs(Fraction(t))
    best = None
    for c in range(32):
        d = abs(ft - tab[c][0])
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (32 if neg else 0)


def brute_int8_row(w_row):
    """(codes, scale bits) for one fp32 row, by exact arithmetic and search over -127..127."""
    amax = max(abs(Fraction(float(v))) for v in w_row)
    s = fp16_round(amax / 127)
    if s == 0:
        return [0] * len(w_row), 0
    codes = []
    for v in w_row:
        fv = Fraction(float(v))
        best = None
        for q in range(-127, 128):
            d = abs(fv - q * s)
            if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
                best = (d, q)
        codes.append(best[1])
    return codes, fraction_to_f16_bits(s)


def brute_int4_group(w_grp, top=15):
    """(codes, scale bits, zero bits) for one group of 32 fp32 weights; codes 0..top (15 for int4,
    7 for int3)."""
    fw = [Fraction(float(v)) for v in w_grp]
    lo = min(min(fw), Fraction(0))
    hi = max(max(fw), Fraction(0))
    s = fp16_round((hi - lo) / top)
    if s == 0:
        return [0] * len(w_grp), 0, 0
    # zero point: the integer 0..top nearest to -lo/s, ties to even
    best = None
    for z in range(top + 1):
        d = abs(-lo / s - z)
        if best is None or d < best[0] or (d == best[0] and z % 2 == 0):
            best = (d, z)
    z = best[1]
    codes = []
    for fv in fw:
        best = None
        for q in range(top + 1):
            d = abs(fv / s - (q - z))
            if best is None or d < best[0] or (d == best[0] and (q - z) % 2 == 0):
                best = (d, q)
        codes.append(best[1])
    return codes, fraction_to_f16_bits(s), fraction_to_f16_bits(Fraction(z))


def brute_fp6_row(w_row):
    """(codes, scale bits) for one fp32 row: exact quotient w/s, nearest e3m2 magnitude, ties to even code."""
    amax = max(abs(Fraction(float(v))) for v in w_row)
    s = fp16_round(amax / 28)
    if s == 0:
        return [0] * len(w_row), 0
    tab = golden_e3m2()
    codes = []
    for v in w_row:
        a = abs(Fraction(float(v))) / s
        best = None
        for c in range(32):
            d = abs(a - tab[c][0])
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        codes.append(best[1] | (32 if math.copysign(1.0, float(v)) < 0 else 0))
    return codes, fraction_to_f16_bits(s)


def check_quantizer(fmt_name, quant_fn, w):
    """Compare quant_fn(w) with the brute-force exact quantizer on every row (and group)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    out = quant_fn(w)
    if fmt_name == "w8":
        q, s = out
        for r in range(n):
            bq, bs = brute_int8_row(w[r])
            if int(s[r]) != bs or [int(v) for v in q[r]] != bq:
                return False
        return True
    if fmt_name in ("w4", "w3"):
        q, s, z = out
        s = np.asarray(s).reshape(n, k // 32)
        z = np.asarray(z).reshape(n, k // 32)
        for r in range(n):
            for g in range(k // 32):
                bq, bs, bz = brute_int4_group(w[r, 32 * g:32 * g + 32], 15 if fmt_name == "w4" else 7)
                if int(s[r, g]) != bs or int(z[r, g]) != bz:
                    return False
                if [int(v) for v in q[r, 32 * g:32 * g + 32]] != bq:
                    return False
        return True
    if fmt_name in ("w6", "fp4", "fp5"):
        q, s = out
        brute = {"w6": brute_fp6_row, "fp4": brute_fp4_row, "fp5": brute_fp5_row}[fmt_name]
        for r in range(n):
            bq, bs = brute(w[r])
            if int(s[r]) != bs or [int(v) for v in q[r]] != bq:
                return False
        return True
    raise ValueError(fmt_name)


# ---------------------------------------------------------------- packing fixtures
def golden_pack_examples():
    """[(fmt name, codes list, expected bytes)] from tests/golden/pack_examples.txt."""
    out = []
    with open(os.path.join(GOLDEN, "pack_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, codes, hexbytes = [p.strip() for p in line.split("|")]
            if name == "F16":
                cl = [int(t, 16) for t in codes.split()]
            else:
                cl = [int(t) for t in codes.split()]
            out.append((name, cl, bytes(int(t, 16) for t in hexbytes.split())))
    return out


# ---------------------------------------------------------------- exact linear and dequant
def exact_dequant(fmt_name, code, scale_bits, zero_bits=0, act="f16"):
    """Exact dequantized value (Fraction) rounded once to fp16 (or bfloat16), returned as bits."""
    s = f16_bits_to_fraction(scale_bits)
    if fmt_name == "w8":
        v = code * s
    elif fmt_name in ("w4", "w3"):
        v = (code - f16_bits_to_fraction(zero_bits)) * s
    elif fmt_name in ("w6", "p24", "fp4", "fp5"):
        mag, neg = {"w6": golden_e3m2, "p24": golden_e3m2, "fp4": golden_e2m1, "fp5": golden_e2m2}[fmt_name]()[code]
        v = (-mag if neg else mag) * s
        if v == 0:
            return 0x8000 if (neg and s > 0) or (not neg and s < 0) else 0
    else:
        raise ValueError(fmt_name)
    r = fp16_round(v) if act == "f16" else bf16_round(v)
    if r == 0:
        return 0x8000 if v < 0 else 0
    return fraction_to_f16_bits(r) if act == "f16" else fraction_to_bf16_bits(r)


def exact_linear(x_bits, w_bits, value=f16_bits_to_fraction):
    """y[m][n] = sum_k x*w as exact Fractions, by a plain triple loop."""
    m, k = x_bits.shape
    n = w_bits.shape[0]
    y = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                acc += value(x_bits[i, t]) * value(w_bits[j, t])
            y[i][j] = acc
    return y


def check_linear(linear_fn, x_bits, w_bits, value=f16_bits_to_fraction):
    """linear_fn(x, w) (float64) must equal the exact sum to within float64 rounding."""
    y = np.asarray(linear_fn(x_bits, w_bits), dtype=np.float64)
    ye = exact_linear(x_bits, w_bits, value)
    if y.shape != (x_bits.shape[0], w_bits.shape[0]):
        return False
    k = x_bits.shape[1]
    for i in range(y.shape[0]):
        for j in range(y.shape[1]):
            mag = sum(abs(value(x_bits[i, t]) * value(w_bits[j, t])) for t in range(k))
            if abs(Fraction(float(y[i, j])) - ye[i][j]) > mag * Fraction(k + 1, 2 ** 52):
                return False
    return True


# ---------------------------------------------------------------- decode-step components
def golden_decode_examples():
    """Parsed tests/golden/decode_examples.txt: {name: (inputs dict of strings, expected floats)}."""
    out = {}
    with open(os.path.join(GOLDEN, "decode_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, ins, exp = [p.strip() for p in line.split("|")]
            kv = dict(item.split("=", 1) for item in ins.split())
            out[name] = (kv, [float(v) for v in exp.split()])
    return out


def _vec(s):
    return np.array([float(v) for v in s.split(",")])


def check_rmsnorm(fn):
    """fn(x [M,d], g [d], eps) against the hand-derived examples."""
    ex = golden_decode_examples()
    for name in ("rmsnorm", "rmsnorm_eps"):
        kv, want = ex[name]
        got = fn(_vec(kv["x"])[None, :], _vec(kv["g"]), float(kv["eps"]))[0]
        if not np.allclose(got, want, rtol=2e-3, atol=0):    # the function rounds to fp16
            return False
    return True


def check_rope(fn):
    """fn(x [M, heads*hd], pos, hd, theta) against the hand-derived examples, plus two exact facts:
    position 0 is the identity and every pair keeps its length."""
    ex = golden_decode_examples()
    for name in ("rope", "rope_pos2"):
        kv, want = ex[name]
        got = fn(_vec(kv["x"])[None, :], int(kv["pos"]), int(kv["hd"]), float(kv["theta"]))[0]
        if not np.allclose(got, want, rtol=1e-11, atol=1e-12):
            return False
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3 * 8))
    if not np.array_equal(fn(x, 0, 8, 10000.0), x):
        return False
    y = fn(x, 37, 8, 10000.0)
    n0 = x.reshape(2, 3, 4, 2) ** 2
    n1 = y.reshape(2, 3, 4, 2) ** 2
    return bool(np.allclose(n0.sum(-1), n1.sum(-1), rtol=1e-12))


def check_attention(fn):
    """fn(q, cache_k, cache_v, pos, n_heads, n_kv_heads, hd) against the hand-derived example, the
    one-position case (the output is that position's value), a library softmax (scipy) on random
    data with grouped heads, and equal scores (the mean of the values)."""
    from scipy.special import softmax
    kv, want = golden_decode_examples()["attention"]
    q = _vec(kv["q"])[None, :]
    k = np.array([_vec(r) for r in kv["k"].split(";")])[None]
    v = np.array([_vec(r) for r in kv["v"].split(";")])[None]
    if not np.allclose(fn(q, k, v, 1, 1, 1, 2)[0], want, rtol=1e-8):
        return False
    rng = np.random.default_rng(9)
    H, Hkv, hd, S, pos = 4, 2, 8, 6, 4
    q = rng.standard_normal((2, H * hd))
    ck, cv = rng.standard_normal((2, S, Hkv * hd)), rng.standard_normal((2, S, Hkv * hd))
    if not np.allclose(fn(q, ck, cv, 0, H, Hkv, hd)[:, :hd], cv[:, 0, :hd], rtol=1e-13):
        return False
    got = fn(q, ck, cv, pos, H, Hkv, hd)
    for b in range(2):
        for h in range(H):
            kvh = h // (H // Hkv)
            s = ck[b, :pos + 1, kvh * hd:(kvh + 1) * hd] @ q[b, h * hd:(h + 1) * hd] / np.sqrt(hd)
            ref = softmax(s) @ cv[b, :pos + 1, kvh * hd:(kvh + 1) * hd]
            if not np.allclose(got[b, h * hd:(h + 1) * hd], ref, rtol=1e-12, atol=1e-14):
                return False
    z = fn(np.zeros((1, hd)), ck[:1, :, :hd], cv[:1, :, :hd], pos, 1, 1, hd)
    return bool(np.allclose(z[0], cv[0, :pos + 1, :hd].mean(axis=0), rtol=1e-12))


def check_silu_mul(fn):
    """fn(g, u) against the hand-derived example and scipy's logistic function."""
    from scipy.special import expit
    kv, want = golden_decode_examples()["silu_mul"]
    if not np.allclose(fn(np.array([float(kv["g"])]), np.array([float(kv["u"])])), want, rtol=1e-3):
        return False
    g = np.linspace(-12, 12, 97)
    u = np.cos(g)
    ref = g * expit(g) * u
    return bool(np.allclose(fn(g, u), ref, rtol=2 ** -10, atol=2 ** -24))


def check_argmax(fn):
    """fn(logits [M, V]) -> the lowest index of the largest value per row."""
    x = np.array([[1.0, 3.0, 3.0, 2.0], [-1.0, -1.0, -2.0, -1.0], [0.0, 0.0, 0.0, 5.0]])
    return bool(np.array_equal(fn(x), [1, 0, 3]))
