"""Pins of the CPU oracle against closed forms, brute force, exact arithmetic and hand-typed fixtures."""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import (FMT_F16, FMT_W8, FMT_W4G32, FMT_W6E3M2, FMT_W4E2M1, FMT_BF16, FMT_W5E2M2, FMT_W3G32,
                    FMT_W6E3M2_P24)
from tests import pins

FMTS = {"w8": FMT_W8, "w4": FMT_W4G32, "w6": FMT_W6E3M2, "f16": FMT_F16, "fp4": FMT_W4E2M1, "bf16": FMT_BF16,
        "fp5": FMT_W5E2M2, "w3": FMT_W3G32, "p24": FMT_W6E3M2_P24}


# ------------------------------------------------------------------ e3m2
def test_e3m2_table_matches_hand_typed_table():
    assert pins.check_e3m2_table(oracle.e3m2_value)


def test_e3m2_special_values():
    t = oracle.e3m2_table()
    assert t[31] == 28.0 and t[63] == -28.0                # largest magnitude, no inf/NaN
    assert t[1] == 0.0625                                   # smallest subnormal 2^-4
    assert t[4] == 0.25                                     # smallest normal 2^(1-3)
    assert t[0] == 0.0 and not math.copysign(1, t[0]) < 0
    assert t[32] == 0.0 and math.copysign(1, t[32]) < 0     # -0
    assert len(set(t.tolist())) == 63                       # +0 and -0 compare equal
    assert np.all(np.diff(t[:32]) > 0)                      # magnitudes increase with the code
    assert np.array_equal(t[32:], -t[:32])
    assert np.all(np.isfinite(t))


def test_e3m2_fp16_bit_placement_identity():
    # code bits s.eee.mm placed at fp16 bits 15 and 12..8 give e3m2(c) * 2^-12 exactly,
    # subnormals and -0 included (fp16 exponent bias 15 = e3m2 bias 3 + 12)
    for c in range(64):
        bits = ((c & 0x20) << 10) | ((c & 0x1F) << 8)
        v = float(np.uint16(bits).view(np.float16))
        assert v * 4096.0 == oracle.e3m2_value(c)
        assert math.copysign(1, v) == math.copysign(1, oracle.e3m2_value(c))


@pytest.mark.parametrize("t,code", [
    (1.875, 16), (-1.875, 48),        # tie between 1.75 (code 15) and 2.0 (code 16): even code
    (0.03125, 0), (-0.03125, 32),     # tie between 0 and 1/16: code 0, sign kept
    (0.09375, 2),                     # tie between 1/16 (code 1) and 1/8 (code 2)
    (26.0, 30), (27.0, 31), (28.0, 31), (1e6, 31), (-1e6, 63),
    (-1e-9, 32), (-0.0, 32), (0.0, 0),
    (0.2, 3), (0.22, 4), (5.5, 22), (5.4999, 21), (5.5001, 22),
])
def test_e3m2_encode_examples(t, code):
    assert int(oracle.e3m2_encode(np.array([t]))[0]) == code


def test_e3m2_encode_vs_exact_brute_force():
    rng = np.random.default_rng(7)
    tab = oracle.e3m2_table()
    mids = [(tab[c] + tab[c + 1]) / 2 for c in range(31)]
    vals = list(rng.standard_normal(2000) * 6) + mids + [-m for m in mids]
    vals += [m + d for m in mids for d in (1e-12, -1e-12)]
    vals += [tab[c] for c in range(64)] + [30.0, -29.0, 28.5, 1e-30, -1e-30]
    got = oracle.e3m2_encode(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == pins.brute_fp6_code(float(v)), v


# ------------------------------------------------------------------ e2m1 (FP4)
def test_e2m1_table_matches_hand_typed_table():
    assert pins.check_e2m1_table(oracle.e2m1_value)


def test_e2m1_special_values():
    t = oracle.e2m1_table()
    assert t[7] == 6.0 and t[15] == -6.0                    # largest magnitude, no inf/NaN
    assert t[1] == 0.5                                      # the one subnormal, 2^(1-1) / 2
    assert t[2] == 1.0                                      # smallest normal
    assert t[0] == 0.0 and not math.copysign(1, t[0]) < 0
    assert t[8] == 0.0 and math.copysign(1, t[8]) < 0       # -0
    assert np.all(np.diff(t[:8]) > 0)
    assert np.array_equal(t[8:], -t[:8])


def test_e2m1_fp16_bit_placement_identity():
    # code bits s.ee.m placed at fp16 bits 15 and 11..9 give e2m1(c) * 2^-14 exactly,
    # the subnormal and -0 included (fp16 exponent bias 15 = e2m1 bias 1 + 14)
    for c in range(16):
        bits = ((c & 0x8) << 12) | ((c & 0x7) << 9)
        v = float(np.uint16(bits).view(np.float16))
        assert v * 16384.0 == oracle.e2m1_value(c)
        assert math.copysign(1, v) == math.copysign(1, oracle.e2m1_value(c))


@pytest.mark.parametrize("t,code", [
    (0.25, 0), (-0.25, 8),            # tie between 0 and 0.5: code 0, sign kept
    (0.75, 2), (1.25, 2), (1.75, 4),  # ties between neighbours go to the even code
    (2.5, 4), (3.5, 6), (5.0, 6),
    (5.01, 7), (6.0, 7), (1e6, 7), (-1e6, 15),
    (-1e-9, 8), (-0.0, 8), (0.0, 0), (0.74, 1), (0.76, 2),
])
def test_e2m1_encode_examples(t, code):
    assert int(oracle.e2m1_encode(np.array([t]))[0]) == code


def test_e2m1_encode_vs_exact_brute_force():
    rng = np.random.default_rng(17)
    tab = oracle.e2m1_table()
    mids = [(tab[c] + tab[c + 1]) / 2 for c in range(7)]
    vals = list(rng.standard_normal(1000) * 3) + mids + [-m for m in mids]
    vals += [m + d for m in mids for d in (1e-12, -1e-12)]
    vals += [tab[c] for c in range(16)] + [7.0, -6.5, 6.01, 1e-30, -1e-30]
    got = oracle.e2m1_encode(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == pins.brute_fp4_code(float(v)), v


# ------------------------------------------------------------------ e2m2 (FP5)
def test_e2m2_table_matches_hand_typed_table():
    assert pins.check_e2m2_table(oracle.e2m2_value)


def test_e2m2_special_values():
    t = oracle.e2m2_table()
    assert t[15] == 7.0 and t[31] == -7.0                   # largest magnitude, no inf/NaN
    assert list(t[1:4]) == [0.25, 0.5, 0.75]                # the subnormals, 2^(1-1) m / 4
    assert t[4] == 1.0                                      # smallest normal
    assert t[0] == 0.0 and not math.copysign(1, t[0]) < 0
    assert t[16] == 0.0 and math.copysign(1, t[16]) < 0     # -0
    assert np.all(np.diff(t[:16]) > 0)
    assert np.array_equal(t[16:], -t[:16])
    # the FP4 values are the even-mantissa FP5 values: e2m1 code s.ee.m is e2m2 code s.ee.m0
    assert all(oracle.e2m2_value(((c & 8) << 1) | ((c & 7) << 1)) == oracle.e2m1_value(c) for c in range(16))


def test_e2m2_fp16_bit_placement_identity():
    # code bits s.ee.mm placed at fp16 bits 15 and 11..8 give e2m2(c) * 2^-14 exactly,
    # the subnormals and -0 included (fp16 exponent bias 15 = e2m2 bias 1 + 14)
    for c in range(32):
        bits = ((c & 0x10) << 11) | ((c & 0xF) << 8)
        v = float(np.uint16(bits).view(np.float16))
        assert v * 16384.0 == oracle.e2m2_value(c)
        assert math.copysign(1, v) == math.copysign(1, oracle.e2m2_value(c))


@pytest.mark.parametrize("t,code", [
    (0.125, 0), (-0.125, 16),         # tie between 0 and 0.25: code 0, sign kept
    (0.375, 2), (0.625, 2), (1.125, 4), (1.375, 6), (1.875, 8),   # ties go to the even code
    (2.25, 8), (2.75, 10), (3.75, 12), (4.5, 12), (5.5, 14), (6.5, 14),
    (6.51, 15), (7.0, 15), (1e6, 15), (-1e6, 31),
    (-1e-9, 16), (-0.0, 16), (0.0, 0), (0.374, 1), (0.376, 2),
])
def test_e2m2_encode_examples(t, code):
    assert int(oracle.e2m2_encode(np.array([t]))[0]) == code


def test_e2m2_encode_vs_exact_brute_force():
    rng = np.random.default_rng(19)
    tab = oracle.e2m2_table()
    mids = [(tab[c] + tab[c + 1]) / 2 for c in range(15)]
    vals = list(rng.standard_normal(1000) * 3) + mids + [-m for m in mids]
    vals += [m + d for m in mids for d in (1e-12, -1e-12)]
    vals += [tab[c] for c in range(32)] + [8.0, -7.5, 7.01, 1e-30, -1e-30]
    got = oracle.e2m2_encode(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == pins.brute_fp5_code(float(v)), v


# ------------------------------------------------------------------ fp16 rounding
def test_fp16_rounding_vs_exact():
    rng = np.random.default_rng(3)
    vals = list(rng.standard_normal(500) * 1e-3) + list(rng.standard_normal(500) * 100)
    vals += [65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 1 + 2.0 ** -11,
             1 + 3 * 2.0 ** -11, 0.1 / 127, 1e-9, -1e-5]
    got = oracle.fp16_bits(np.array(vals))
    for v, g in zip(vals, got):
        r = pins.fp16_round(Fraction(v))
        assert int(g) == pins.fraction_to_f16_bits(r) or (r == 0 and int(g) in (0, 0x8000)), v


# ------------------------------------------------------------------ bfloat16 rounding
def _bf16_probe_values(rng):
    vals = list(rng.standard_normal(400) * 1e-3) + list(rng.standard_normal(400) * 300)
    vals += [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8 - 2.0 ** -40,   # ties, near-ties
             2 - 2.0 ** -9, 2 - 2.0 ** -10, -(1 + 5 * 2.0 ** -8),
             2.0 ** -126, 2.0 ** -127 + 2.0 ** -134, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -135,
             -(2.0 ** -134),                                                     # rounds to -0
             (2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127,          # largest; the tie above it -> inf
             (2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -40), 1e39, -1e39,
             0.1, -0.1, 1e-40, -3.5e-39, 65504.0, 1e30, 0.0, -0.0]
    return vals


def test_bf16_rounding_vs_exact():
    assert pins.check_bf16_rounding(oracle.bf16_bits, _bf16_probe_values(np.random.default_rng(5)))


def test_bf16_rounding_vs_torch_float32_conversion():
    # torch rounds float32 to bfloat16 to nearest, ties to even, in one step: a library routine
    import torch
    rng = np.random.default_rng(6)
    f = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    ties = ((rng.integers(0, 2 ** 16, 4000, dtype=np.uint64).astype(np.uint32) << np.uint32(16))
            | np.uint32(0x8000)).view(np.float32)                  # exactly half way, both parities of the last bit
    f = np.concatenate([f, ties])
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits(f.astype(np.float64)), want)


def test_bf16_from_bits_matches_the_fields():
    for b in list(range(0, 0x7F80, 97)) + [0x0001, 0x007F, 0x0080, 0x3F80, 0x7F7F]:
        for sb in (b, b | 0x8000):
            v = oracle.bf16_from_bits(np.array([sb], dtype=np.uint16))[0]
            assert Fraction(float(v)) == pins.bf16_bits_to_fraction(sb), hex(sb)
            assert int(oracle.bf16_bits(np.array([v]))[0]) == sb or (v == 0 and sb in (0, 0x8000))


# ------------------------------------------------------------------ quantizers
def _adversarial(n, k, rng):
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[0, :] = 0.0                                              # all-zero row -> scale 0
    w[1, 5] = 0.5                                              # one large weight
    w[2, :] = np.abs(w[2, :])                                  # one-signed row
    w[3, :] = -np.abs(w[3, :])
    w[4, :32] = 1e-9                                           # group whose scale is subnormal
    w[5, 7] = -0.0
    return w


@pytest.mark.parametrize("name", ["w8", "w4", "w6", "fp4", "fp5", "w3"])
def test_quantizer_vs_brute_force(name):
    rng = np.random.default_rng(11)
    w = _adversarial(8, 64, rng)
    fn = {"w8": oracle.quantize_int8, "w4": oracle.quantize_int4_g32, "w6": oracle.quantize_fp6,
          "fp4": oracle.quantize_fp4, "fp5": oracle.quantize_fp5, "w3": oracle.quantize_int3_g32}[name]
    assert pins.check_quantizer(name, fn, w)


def test_int8_ties_round_to_even():
    # scale 1 exactly (max |w| = 127); w = 2.5 -> 2, 3.5 -> 4, -2.5 -> -2
    w = np.array([[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5] + [0.0] * 24], dtype=np.float32)
    q, s = oracle.quantize_int8(w)
    assert int(s[0]) == 0x3C00
    assert q[0, :8].tolist() == [127, 2, 4, -2, -4, 0, 0, 126]


def test_int8_never_minus_128():
    w = np.array([[-1.0] * 31 + [1.0 - 2 ** -20]], dtype=np.float32)
    q, _ = oracle.quantize_int8(w)
    assert q.min() == -127


def test_int4_zero_point_and_range():
    # group spanning [-1, 2]: s = fp16(3/15) = fp16(0.2), z = rint(1/s) = 5
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0], w[0, 1] = -1.0, 2.0
    q, s, z = oracle.quantize_int4_g32(w)
    sv = float(np.uint16(s[0, 0]).view(np.float16))
    assert sv == float(np.float16(0.2))
    assert float(np.uint16(z[0, 0]).view(np.float16)) == 5.0
    assert q[0, 0] == 0 and q[0, 1] == 15 and q[0, 2] == 5    # 0 maps to the zero point


def test_int3_zero_point_and_range():
    # group spanning [-1, 2.5]: s = fp16(3.5/7) = 0.5 exactly, z = rint(1/0.5) = 2;
    # 0.25 / 0.5 = 0.5 is a tie: rint -> 0, code 2; 0.75 / 0.5 = 1.5 -> 2, code 4
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0], w[0, 1], w[0, 3], w[0, 4] = -1.0, 2.5, 0.25, 0.75
    q, s, z = oracle.quantize_int3_g32(w)
    assert int(s[0, 0]) == 0x3800                             # fp16 0.5
    assert float(np.uint16(z[0, 0]).view(np.float16)) == 2.0
    assert q[0, :5].tolist() == [0, 7, 2, 2, 4]
    # all-positive group: lo = 0, z = 0, the largest weight takes code 7
    w = np.linspace(0.0, 7.0, 32, dtype=np.float32).reshape(1, 32)
    q, s, z = oracle.quantize_int3_g32(w)
    assert int(z[0, 0]) == 0 and q[0, 0] == 0 and q[0, 31] == 7


def test_fp6_saturation_and_negative_zero():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 28.0          # scale 1
    w[0, 1] = -28.0
    w[0, 2] = -0.001        # rounds to -0
    w[0, 3] = 1.875         # tie -> 2.0
    codes, s = oracle.quantize_fp6(w)
    assert int(s[0]) == 0x3C00
    assert codes[0, :4].tolist() == [31, 63, 32, 16]


def test_fp4_saturation_and_negative_zero():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 6.0           # scale 1
    w[0, 1] = -6.0
    w[0, 2] = -0.001        # rounds to -0
    w[0, 3] = 2.5           # tie between 2 (code 4) and 3 (code 5) -> 4
    w[0, 4] = 0.25          # tie between 0 and 0.5 -> 0
    codes, s = oracle.quantize_fp4(w)
    assert int(s[0]) == 0x3C00
    assert codes[0, :5].tolist() == [7, 15, 8, 4, 0]


def test_fp5_saturation_and_negative_zero():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 7.0           # scale 1
    w[0, 1] = -7.0
    w[0, 2] = -0.001        # rounds to -0
    w[0, 3] = 4.5           # tie between 4 (code 12) and 5 (code 13) -> 12
    w[0, 4] = 0.125         # tie between 0 and 0.25 -> 0
    w[0, 5] = 0.625         # tie between 0.5 (code 2) and 0.75 (code 3) -> 2
    codes, s = oracle.quantize_fp5(w)
    assert int(s[0]) == 0x3C00
    assert codes[0, :6].tolist() == [15, 31, 16, 12, 0, 2]


def test_quantizer_errors():
    with pytest.raises(oracle.OracleRangeError):
        oracle.quantize_int8(np.array([[np.nan] * 32], dtype=np.float32))
    with pytest.raises(oracle.OracleRangeError):
        oracle.quantize_fp6(np.array([[1e7] * 32], dtype=np.float32))     # 1e7/28 overflows fp16


# ------------------------------------------------------------------ layout
def test_pack_matches_hand_derived_bytes():
    for name, codes, expected in pins.golden_pack_examples():
        fmt = FMTS[name.lower().split("x")[0]]
        c = np.array([codes])
        assert bytes(oracle.pack_scalar(fmt, c)) == expected, name
        assert bytes(oracle.pack_vectorized(fmt, c)) == expected, name


@pytest.mark.parametrize("name", ["w8", "w4", "w6", "f16", "fp4", "bf16", "fp5", "w3", "p24"])
@pytest.mark.parametrize("n,k", [(3, 96), (2, 32 * 130)])       # 130 units: two full chunks of 64 and one of 2
def test_pack_scalar_equals_vectorized_and_round_trips(name, n, k):
    fmt = FMTS[name]
    rng = np.random.default_rng(5)
    if name == "w8":
        codes = rng.integers(-127, 128, (n, k)).astype(np.int8)
    elif name in ("w4", "fp4"):
        codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    elif name in ("w6", "p24"):
        codes = rng.integers(0, 64, (n, k)).astype(np.uint8)
    elif name == "fp5":
        codes = rng.integers(0, 32, (n, k)).astype(np.uint8)
    elif name == "w3":
        codes = rng.integers(0, 8, (n, k)).astype(np.uint8)
    else:
        codes = rng.integers(0, 65536, (n, k)).astype(np.uint16)
    a = oracle.pack_scalar(fmt, codes)
    b = oracle.pack_vectorized(fmt, codes)
    assert a.size == oracle.packed_bytes(fmt, n, k) == n * k * {"w8": 8, "w4": 4, "w6": 6, "f16": 16, "fp4": 4,
                                                                "bf16": 16, "fp5": 5, "w3": 3, "p24": 6}[name] // 8
    assert np.array_equal(a, b)
    assert np.array_equal(oracle.unpack_scalar(fmt, a, n, k), codes)
    assert np.array_equal(oracle.unpack_vectorized(fmt, b, n, k), codes)


def test_metadata_counts():
    assert oracle.scales_count(FMT_W8, 7, 64) == 7 and oracle.zeros_count(FMT_W8, 7, 64) == 0
    assert oracle.scales_count(FMT_W6E3M2, 7, 64) == 7
    assert oracle.scales_count(FMT_W4G32, 7, 64) == 14 and oracle.zeros_count(FMT_W4G32, 7, 64) == 14
    assert oracle.scales_count(FMT_F16, 7, 64) == 0
    assert oracle.scales_count(FMT_W4E2M1, 7, 64) == 7 and oracle.zeros_count(FMT_W4E2M1, 7, 64) == 0
    assert oracle.scales_count(FMT_BF16, 7, 64) == 0 and oracle.zeros_count(FMT_BF16, 7, 64) == 0
    assert oracle.scales_count(FMT_W5E2M2, 7, 64) == 7 and oracle.zeros_count(FMT_W5E2M2, 7, 64) == 0
    assert oracle.scales_count(FMT_W3G32, 7, 64) == 14 and oracle.zeros_count(FMT_W3G32, 7, 64) == 14
    assert oracle.scales_count(FMT_W6E3M2_P24, 7, 64) == 7 and oracle.zeros_count(FMT_W6E3M2_P24, 7, 64) == 0


def test_p24_holds_the_w6_codes():
    # the 2+4 split stores the same e3m2 codes and scales as W6; only the bytes differ
    rng = np.random.default_rng(23)
    w = rng.standard_normal((5, 32 * 67)).astype(np.float32)
    pa, sa, za, ca = oracle.quantize_and_pack(FMT_W6E3M2, w)
    pb, sb, zb, cb = oracle.quantize_and_pack(FMT_W6E3M2_P24, w)
    assert np.array_equal(ca, cb) and np.array_equal(sa, sb) and pa.size == pb.size
    assert not np.array_equal(pa, pb)
    assert np.array_equal(oracle.unpack_vectorized(FMT_W6E3M2_P24, pb, 5, 32 * 67), ca)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("name", ["w8", "w4", "w6", "fp4", "fp5", "w3", "p24"])
def test_dequant_exact_vs_fraction_and_fp32(name):
    fmt = FMTS[name]
    rng = np.random.default_rng(9)
    w = _adversarial(8, 64, rng)
    w[6, :] *= 1e-4                                    # small scales: subnormal products
    packed, s, z, codes = oracle.quantize_and_pack(fmt, w)
    d = oracle.dequant_fp16(fmt, codes, s, z)
    n, k = codes.shape
    sv = np.asarray(s).reshape(n, -1)
    grouped = name in ("w4", "w3")
    zv = np.asarray(z).reshape(n, -1) if grouped else None
    for r in range(n):
        for c in range(k):
            g = c // 32 if grouped else 0
            want = pins.exact_dequant(name, int(codes[r, c]), int(sv[r, g]), int(zv[r, g]) if zv is not None else 0)
            got = int(d[r, c])
            assert got == want or (want in (0, 0x8000) and got in (0, 0x8000) and
                                   name not in ("w6", "p24", "fp4", "fp5")), (r, c)
    # the product is exact in fp32 as well, so an fp32 multiply then one rounding agrees bit for bit
    s32 = oracle.fp16_from_bits(sv).astype(np.float32)
    if name == "w8":
        v32 = codes.astype(np.float32) * np.repeat(s32, k, axis=1)
    elif grouped:
        zz = oracle.fp16_from_bits(zv).astype(np.float32)
        v32 = (codes.astype(np.float32) - np.repeat(zz, 32, axis=1)) * np.repeat(s32, 32, axis=1)
    elif name in ("w6", "p24"):
        v32 = oracle.e3m2_table().astype(np.float32)[codes] * np.repeat(s32, k, axis=1)
    elif name == "fp5":
        v32 = oracle.e2m2_table().astype(np.float32)[codes] * np.repeat(s32, k, axis=1)
    else:
        v32 = oracle.e2m1_table().astype(np.float32)[codes] * np.repeat(s32, k, axis=1)
    assert np.array_equal(v32.astype(np.float16).view(np.uint16), d)


@pytest.mark.parametrize("name", ["w8", "w4", "w6", "fp4", "fp5"])
def test_dequant_bf16_exact_vs_fraction_and_fp32(name):
    import torch
    fmt = FMTS[name]
    rng = np.random.default_rng(19)
    w = _adversarial(8, 64, rng)
    w[6, :] *= 1e-4
    _, s, z, codes = oracle.quantize_and_pack(fmt, w)
    d = oracle.dequant_bf16(fmt, codes, s, z)
    n, k = codes.shape
    sv = np.asarray(s).reshape(n, -1)
    zv = np.asarray(z).reshape(n, -1) if name == "w4" else None
    for r in range(n):
        for c in range(k):
            g = c // 32 if name == "w4" else 0
            want = pins.exact_dequant(name, int(codes[r, c]), int(sv[r, g]), int(zv[r, g]) if zv is not None else 0,
                                      act="bf16")
            got = int(d[r, c])
            assert got == want or (want in (0, 0x8000) and got in (0, 0x8000) and name not in ("w6", "fp4", "fp5")), (r, c)
    # exact in fp32 too: an fp32 product rounded once by torch gives the same bits
    s32 = oracle.fp16_from_bits(sv).astype(np.float32)
    if name == "w8":
        v32 = codes.astype(np.float32) * np.repeat(s32, k, axis=1)
    elif name == "w4":
        zz = oracle.fp16_from_bits(zv).astype(np.float32)
        v32 = (codes.astype(np.float32) - np.repeat(zz, 32, axis=1)) * np.repeat(s32, 32, axis=1)
    elif name == "w6":
        v32 = oracle.e3m2_table().astype(np.float32)[codes] * np.repeat(s32, k, axis=1)
    elif name == "fp5":
        v32 = oracle.e2m2_table().astype(np.float32)[codes] * np.repeat(s32, k, axis=1)
    else:
        v32 = oracle.e2m1_table().astype(np.float32)[codes] * np.repeat(s32, k, axis=1)
    t = torch.from_numpy(np.ascontiguousarray(v32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, d)


def test_dequant_w6_keeps_negative_zero():
    codes = np.full((1, 32), 32, dtype=np.uint8)
    d = oracle.dequant_fp16(FMT_W6E3M2, codes, np.array([0x3C00], dtype=np.uint16))
    assert np.all(d == 0x8000)


# ------------------------------------------------------------------ linear
@pytest.mark.parametrize("m,n,k", [(1, 3, 32), (2, 5, 64), (2, 8, 32)])
def test_linear_vs_exact_triple_loop(m, n, k):
    rng = np.random.default_rng(m * 100 + n)
    x = rng.standard_normal((m, k)).astype(np.float16).view(np.uint16)
    w = (rng.standard_normal((n, k)) * 0.1).astype(np.float16).view(np.uint16)
    assert pins.check_linear(oracle.linear_ref, x, w)


@pytest.mark.parametrize("m,n,k", [(1, 3, 32), (2, 5, 64)])
def test_linear_bf16_vs_exact_triple_loop(m, n, k):
    rng = np.random.default_rng(m * 100 + n + 7)
    x = oracle.bf16_bits(rng.standard_normal((m, k)) * 3)
    w = oracle.bf16_bits(rng.standard_normal((n, k)) * 0.1)
    fn = lambda a, b: oracle.linear_ref(a, b, act=oracle.ACT_BF16)
    assert pins.check_linear(fn, x, w, value=pins.bf16_bits_to_fraction)


def test_linear_one_hot_returns_a_column():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((6, 64)) * 0.1).astype(np.float16).view(np.uint16)
    for k in (0, 17, 63):
        x = np.zeros((1, 64), dtype=np.float16)
        x[0, k] = 1.0
        y = oracle.linear_ref(x.view(np.uint16), w)
        assert np.array_equal(y[0], oracle.fp16_from_bits(w[:, k]))


def test_linear_rows_are_independent():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64)).astype(np.float16).view(np.uint16)
    w = (rng.standard_normal((7, 64)) * 0.1).astype(np.float16).view(np.uint16)
    y = oracle.linear_ref(x, w)
    for i in range(5):
        yi = oracle.linear_ref(x[i:i + 1], w)[0]
        assert np.allclose(yi, y[i], rtol=1e-14, atol=1e-14)
    assert np.all(oracle.linear_ref(np.zeros((1, 64), dtype=np.uint16), w) == 0)


def test_error_bound_accepts_fp32_accumulation_and_rejects_one_code_off():
    rng = np.random.default_rng(4)
    n, k = 16, 4096
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = rng.standard_normal((1, k)).astype(np.float16).view(np.uint16)
    _, s, _, codes = oracle.quantize_and_pack(FMT_W8, w)
    wd = oracle.dequant_fp16(FMT_W8, codes, s)
    yref = oracle.linear_ref(x, wd)
    bound = oracle.error_bound(x, wd, yref)
    # an fp32 sum of exact products, scale applied after, summed in a shuffled order
    xf = oracle.fp16_from_bits(x).astype(np.float32)[0]
    for r in range(n):
        order = rng.permutation(k)
        acc = np.float32(0)
        for t in order:
            acc = np.float32(acc + np.float32(xf[t] * np.float32(codes[r, t])))
        y = np.float16(np.float32(acc * np.float32(oracle.fp16_from_bits(s[r]))))
        assert abs(float(y) - yref[0, r]) <= bound[0, r]
    # one code off in one weight, seen through a one-hot x, is far outside the bound
    xo = np.zeros((1, k), dtype=np.float16)
    xo[0, 10] = 1.0
    xo = xo.view(np.uint16)
    yo = oracle.linear_ref(xo, wd)
    bo = oracle.error_bound(xo, wd, yo)
    off = float(oracle.fp16_from_bits(s[0])) * (int(codes[0, 10]) + 1)
    assert abs(off - yo[0, 0]) > bo[0, 0]


def test_error_bound_bf16_accepts_fp32_accumulation_and_rejects_one_code_off():
    # W4 with bfloat16 activations: the group scale applied after each group's fp32 sum, the
    # output rounded once to bfloat16, against the reference on bfloat16-dequantised weights
    rng = np.random.default_rng(14)
    n, k = 16, 4096
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = oracle.bf16_bits(rng.standard_normal((1, k)) * 2)
    _, s, z, codes = oracle.quantize_and_pack(FMT_W4G32, w)
    wd = oracle.dequant_bf16(FMT_W4G32, codes, s, z)
    yref = oracle.linear_ref(x, wd, act=oracle.ACT_BF16)
    bound = oracle.error_bound(x, wd, yref, act=oracle.ACT_BF16)
    assert np.all(bound < oracle.error_bound(x, wd, yref) * 16)          # looser than fp16 by about 2^3
    xf = oracle.bf16_from_bits(x).astype(np.float32)[0]
    sv = oracle.fp16_from_bits(s).reshape(n, k // 32).astype(np.float32)
    zv = oracle.fp16_from_bits(z).reshape(n, k // 32).astype(np.float32)
    for r in range(n):
        acc = np.float32(0)
        for g in rng.permutation(k // 32):
            part = np.float32(0)
            for t in range(32 * g, 32 * g + 32):
                part = np.float32(part + np.float32(xf[t] * np.float32(np.float32(codes[r, t]) - zv[r, g])))
            acc = np.float32(acc + np.float32(part * sv[r, g]))
        y = float(oracle.bf16_from_bits(oracle.bf16_bits(np.array([float(acc)])))[0])
        assert abs(y - yref[0, r]) <= bound[0, r]
    # a weight one code off, seen through a one-hot x, is far outside the bound
    xo = np.zeros((1, k))
    xo[0, 10] = 1.0
    xo = oracle.bf16_bits(xo)
    yo = oracle.linear_ref(xo, wd, act=oracle.ACT_BF16)
    bo = oracle.error_bound(xo, wd, yo, act=oracle.ACT_BF16)
    off = float(sv[0, 0]) * (int(codes[0, 10]) + 1 - float(zv[0, 0]))
    assert abs(off - yo[0, 0]) > bo[0, 0]
