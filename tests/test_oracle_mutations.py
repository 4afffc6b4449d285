"""Planted mistakes: each is a plausible bug in a copy of an oracle function, and a pin must reject it.

The mistakes live only in this file, on the CPU. They show that the pins in
test_oracle_pins.py would notice a dropped term, a wrong sign or index, a wrong tie
rule or a transposed operand, rather than agreeing with whatever the oracle computes.
"""

import numpy as np

import oracle
from oracle import FMT_W4G32, FMT_W6E3M2, FMT_W3G32, FMT_W6E3M2_P24
from tests import pins
from tests.test_oracle_pins import _adversarial, _bf16_probe_values


def test_pins_accept_the_oracle():
    assert pins.check_e3m2_table(oracle.e3m2_value)
    rng = np.random.default_rng(11)
    w = _adversarial(8, 64, rng)
    assert pins.check_quantizer("w8", oracle.quantize_int8, w)
    assert pins.check_quantizer("w4", oracle.quantize_int4_g32, w)
    assert pins.check_quantizer("w6", oracle.quantize_fp6, w)
    assert pins.check_e2m1_table(oracle.e2m1_value)
    assert pins.check_quantizer("fp4", oracle.quantize_fp4, w)
    assert pins.check_e2m2_table(oracle.e2m2_value)
    assert pins.check_quantizer("fp5", oracle.quantize_fp5, w)
    assert pins.check_quantizer("w3", oracle.quantize_int3_g32, w)


def test_int3_with_the_int4_divisor_is_caught():
    def bad_quant(w):   # the int4 rule (15 steps) clamped to 0..7
        q, s, z = oracle.quantize_int4_g32(w)
        return np.minimum(q, 7), s, np.minimum(oracle.fp16_from_bits(z), 7).astype(np.float16).view(np.uint16)
    rng = np.random.default_rng(11)
    assert not pins.check_quantizer("w3", bad_quant, _adversarial(8, 64, rng))


def test_int3_codes_truncated_is_caught():
    def bad_quant(w):   # codes rounded toward zero instead of to nearest
        q, s, z = oracle.quantize_int3_g32(w)
        n, k = w.shape
        sv = oracle.fp16_from_bits(s).reshape(n, k // 32, 1)
        zv = oracle.fp16_from_bits(z).reshape(n, k // 32, 1)
        g = w.astype(np.float64).reshape(n, k // 32, 32)
        q2 = np.clip(np.trunc(g / np.where(sv > 0, sv, 1)) + zv, 0, 7).astype(np.uint8)
        return q2.reshape(n, k), s, z
    rng = np.random.default_rng(11)
    assert not pins.check_quantizer("w3", bad_quant, _adversarial(8, 64, rng))


def test_e2m2_wrong_bias_is_caught():
    assert not pins.check_e2m2_table(lambda c: oracle.e2m2_value(c) * 2)


def test_e2m2_subnormal_as_normal_is_caught():
    def bad(c):
        e, m = (c >> 2) & 3, c & 3
        v = (1 + m / 4) * 2.0 ** (e - 1)          # forgets that exponent field 0 is subnormal
        return -v if c & 16 else v
    assert not pins.check_e2m2_table(bad)


def test_e2m2_mantissa_bits_swapped_is_caught():
    def bad(c):
        return oracle.e2m2_value((c & 0x1C) | ((c & 1) << 1) | ((c >> 1) & 1))
    assert not pins.check_e2m2_table(bad)


def test_fp5_scale_from_fp4_range_is_caught():
    def bad_quant(w):
        w64 = w.astype(np.float64)
        s_bits = oracle.fp16_bits(np.abs(w64).max(axis=1) / 6.0)     # the FP4 maximum, not 7
        s = oracle.fp16_from_bits(s_bits)
        return oracle.e2m2_encode(w64 / s[:, None]), s_bits
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((2, 64)) * 0.1).astype(np.float32)
    assert not pins.check_quantizer("fp5", bad_quant, w)


def test_fp5_sign_plane_order_is_caught():
    for name, codes, expected in pins.golden_pack_examples():
        if name != "FP5":
            continue
        c = np.array(codes, dtype=np.uint32)
        sw = 0
        for j in range(32):                       # signs in code order instead of (even codes, odd codes)
            sw |= int(c[j] >> 4) << j
        assert expected[16:] != sw.to_bytes(4, "little")
        assert expected[16:] == bytes([0x00, 0xFF, 0x00, 0xFF])


def test_e2m1_wrong_bias_is_caught():
    assert not pins.check_e2m1_table(lambda c: oracle.e2m1_value(c) * 2)


def test_e2m1_subnormal_as_normal_is_caught():
    def bad(c):
        e, m = (c >> 1) & 3, c & 1
        v = (1 + m / 2) * 2.0 ** (e - 1)          # forgets that exponent field 0 is subnormal
        return -v if c & 8 else v
    assert not pins.check_e2m1_table(bad)


def test_fp4_ties_away_from_zero_is_caught():
    def bad_quant(w):
        w64 = w.astype(np.float64)
        s_bits = oracle.fp16_bits(np.abs(w64).max(axis=1) / 6.0)
        s = oracle.fp16_from_bits(s_bits)
        t = w64 / s[:, None]
        tab = oracle.e2m1_table()[:8]
        d = np.abs(np.abs(t)[..., None] - tab)
        code = (7 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)   # ties to the larger magnitude
        return code | (np.signbit(t).astype(np.uint8) << 3), s_bits
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 6.0
    w[0, 1:4] = [2.5, 0.25, 5.0]                      # three exact ties (scale is 1)
    assert not pins.check_quantizer("fp4", bad_quant, w)


def test_fp4_swapped_nibbles_are_caught():
    for name, codes, expected in pins.golden_pack_examples():
        if name != "FP4":
            continue
        c = np.array(codes, dtype=np.uint8).reshape(16, 2)
        assert bytes((c[:, 1] | (c[:, 0] << 4)).tolist()) != expected    # code 2p in the high nibble


def test_e3m2_wrong_bias_is_caught():
    assert not pins.check_e3m2_table(lambda c: oracle.e3m2_value(c) / 2)


def test_e3m2_subnormal_as_normal_is_caught():
    def bad(c):
        e, m = (c >> 2) & 7, c & 3
        v = (1 + m / 4) * 2.0 ** (e - 3)          # forgets that exponent field 0 is subnormal
        return -v if c & 32 else v
    assert not pins.check_e3m2_table(bad)


def test_e3m2_lost_negative_zero_is_caught():
    assert not pins.check_e3m2_table(lambda c: 0.0 if c == 32 else oracle.e3m2_value(c))


def test_fp6_ties_away_from_zero_is_caught():
    def bad_quant(w):
        w64 = w.astype(np.float64)
        s_bits = oracle.fp16_bits(np.abs(w64).max(axis=1) / 28.0)
        s = oracle.fp16_from_bits(s_bits)
        t = w64 / s[:, None]
        tab = oracle.e3m2_table()[:32]
        a = np.abs(t)[..., None]
        d = np.abs(a - tab)
        # ties go to the larger magnitude instead of the even code
        code = (31 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)
        return code | (np.signbit(t).astype(np.uint8) << 5), s_bits
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 28.0
    w[0, 1:4] = [1.875, 0.03125, 5.5]                # three exact ties (scale is 1)
    assert not pins.check_quantizer("w6", bad_quant, w)


def test_int4_without_zero_point_is_caught():
    def bad_quant(w):
        q, s, z = oracle.quantize_int4_g32(w)
        n, k = w.shape
        sv = oracle.fp16_from_bits(s).reshape(n, k // 32, 1)
        g = w.astype(np.float64).reshape(n, k // 32, 32)
        q2 = np.clip(np.rint(g / np.where(sv > 0, sv, 1)), 0, 15).astype(np.uint8)   # z dropped
        return q2.reshape(n, k), s, z
    rng = np.random.default_rng(11)
    assert not pins.check_quantizer("w4", bad_quant, _adversarial(8, 64, rng))


def test_int8_wrong_divisor_is_caught():
    def bad_quant(w):
        w64 = w.astype(np.float64)
        s_bits = oracle.fp16_bits(np.abs(w64).max(axis=1) / 128.0)      # 128 instead of 127
        s = oracle.fp16_from_bits(s_bits)
        q = np.clip(np.rint(w64 / np.where(s > 0, s, 1)[:, None]), -127, 127).astype(np.int8)
        return q, s_bits
    rng = np.random.default_rng(11)
    assert not pins.check_quantizer("w8", bad_quant, _adversarial(8, 64, rng))


def test_w4_nibble_order_mistake_is_caught():
    for name, codes, expected in pins.golden_pack_examples():
        if name != "W4":
            continue
        c = np.array([codes], dtype=np.uint32).reshape(1, 4, 8)
        words = np.zeros((1, 4), dtype=np.uint32)
        for p in range(8):
            words |= c[:, :, p] << np.uint32(4 * p)                     # plain order 0..7
        assert words.astype("<u4").tobytes() != expected


def test_w6_big_endian_bit_order_is_caught():
    for name, codes, expected in pins.golden_pack_examples():
        if name != "W6":
            continue
        acc = 0
        for c in codes:                                                  # first code in the top bits
            acc = (acc << 6) | c
        assert acc.to_bytes(24, "little") != expected


def test_linear_transposed_operand_is_caught():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 32)).astype(np.float16).view(np.uint16)
    w = (rng.standard_normal((32, 32)) * 0.1).astype(np.float16).view(np.uint16)   # square: shapes agree
    bad = lambda a, b: oracle.fp16_from_bits(a) @ oracle.fp16_from_bits(b)      # W not transposed
    assert pins.check_linear(oracle.linear_ref, x, w)
    assert not pins.check_linear(bad, x, w)


def test_linear_dropped_term_is_caught():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 32)).astype(np.float16).view(np.uint16)
    w = (rng.standard_normal((4, 32)) * 0.1).astype(np.float16).view(np.uint16)
    bad = lambda a, b: oracle.fp16_from_bits(a)[:, :-1] @ oracle.fp16_from_bits(b)[:, :-1].T
    assert not pins.check_linear(bad, x, w)


def test_dequant_wrong_zero_sign_is_caught():
    rng = np.random.default_rng(9)
    w = _adversarial(8, 64, rng)
    _, s, z, codes = oracle.quantize_and_pack(FMT_W4G32, w)
    good = oracle.dequant_fp16(FMT_W4G32, codes, s, z)
    zz = oracle.fp16_from_bits(z).reshape(8, 2, 1)
    ss = oracle.fp16_from_bits(s).reshape(8, 2, 1)
    bad = oracle.fp16_bits(((codes.reshape(8, 2, 32) + zz) * ss).reshape(8, 64))   # q + z
    r, c = np.argwhere(good != bad)[0]
    want = pins.exact_dequant("w4", int(codes[r, c]), int(s.reshape(8, 2)[r, c // 32]), int(z.reshape(8, 2)[r, c // 32]))
    assert int(good[r, c]) == want and int(bad[r, c]) != want


def test_dequant_w6_sign_dropped_is_caught():
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64)
    s = np.array([0x3C00], dtype=np.uint16)
    good = oracle.dequant_fp16(FMT_W6E3M2, codes, s)
    bad = oracle.fp16_bits(np.abs(oracle.e3m2_table()[codes]))
    mismatches = [c for c in range(64) if int(bad[0, c]) != pins.exact_dequant("w6", c, 0x3C00)]
    assert mismatches and all(int(good[0, c]) == pins.exact_dequant("w6", c, 0x3C00) for c in range(64))


def test_w6_units_stored_whole_is_caught():
    # two units stored one after the other (no planes) must not match the two-unit fixture
    for name, codes, expected in pins.golden_pack_examples():
        if name != "W6x2":
            continue
        whole = b"".join(oracle.pack_scalar(FMT_W6E3M2, np.array([codes[32 * i:32 * i + 32]])).tobytes() for i in range(2))
        assert whole != expected and len(whole) == len(expected)


def test_bf16_truncation_is_caught():
    def bad(a):   # keeps the upper 16 bits of the binary32 value: rounds toward zero
        with np.errstate(over="ignore"):
            f = np.asarray(a, dtype=np.float64).astype(np.float32)
        return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    vals = _bf16_probe_values(np.random.default_rng(5))
    assert pins.check_bf16_rounding(oracle.bf16_bits, vals)
    assert not pins.check_bf16_rounding(bad, vals)


def test_bf16_ties_away_from_zero_is_caught():
    def bad(a):
        a = np.asarray(a, dtype=np.float64)
        _, ex = np.frexp(np.abs(a))
        q = np.ldexp(1.0, np.maximum(ex.astype(np.int64) - 1, -126) - 7)
        r = np.sign(a) * np.floor(np.abs(a) / q + 0.5) * q                 # half away from zero
        return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert not pins.check_bf16_rounding(bad, [1 + 2.0 ** -8, -(1 + 2.0 ** -8), 1.5])


def test_bf16_linear_reading_fp16_bits_is_caught():
    rng = np.random.default_rng(8)
    x = oracle.bf16_bits(rng.standard_normal((1, 32)))
    w = oracle.bf16_bits(rng.standard_normal((3, 32)) * 0.1)
    good = lambda a, b: oracle.linear_ref(a, b, act=oracle.ACT_BF16)
    bad = lambda a, b: oracle.linear_ref(a, b)                         # the bits taken as fp16
    assert pins.check_linear(good, x, w, value=pins.bf16_bits_to_fraction)
    assert not pins.check_linear(bad, x, w, value=pins.bf16_bits_to_fraction)


def test_w3_offsets_in_order_are_caught():
    # pairs at offsets 0, 3, 6, 9, 12 (packed tight, the spread pair elsewhere) must not match the fixture
    for name, codes, expected in pins.golden_pack_examples():
        if name != "W3":
            continue
        c = np.array(codes, dtype=np.uint32).reshape(16, 2)
        words = [0, 0, 0]
        for p in range(15):
            word, f = divmod(p, 5)
            words[word] |= int(c[p, 0]) << (3 * f) | int(c[p, 1]) << (16 + 3 * f)
        for b in range(3):
            words[b] |= ((int(c[15, 0]) >> b) & 1) << 15 | ((int(c[15, 1]) >> b) & 1) << 31
        assert b"".join(w.to_bytes(4, "little") for w in words) != expected


def test_w3_spread_pair_bit_order_is_caught():
    # bit b of the last pair in word 2 - b instead of word b
    for name, codes, expected in pins.golden_pack_examples():
        if name != "W3x1":
            continue
        words = [0, 0, 0]
        for b in range(3):
            words[2 - b] |= ((codes[30] >> b) & 1) << 9 | ((codes[31] >> b) & 1) << 25
        assert b"".join(w.to_bytes(4, "little") for w in words) != expected
        assert expected == bytes(oracle.pack_scalar(FMT_W3G32, np.array([codes])))


def test_p24_planes_swapped_are_caught():
    # the sign word before the bit-4 word must not match the fixture
    for name, codes, expected in pins.golden_pack_examples():
        if name != "P24":
            continue
        good = bytes(oracle.pack_scalar(FMT_W6E3M2_P24, np.array([codes])))
        bad = good[:16] + good[20:24] + good[16:20]
        assert good == expected and bad != expected


def test_p24_units_stored_whole_is_caught():
    for name, codes, expected in pins.golden_pack_examples():
        if name != "P24x2":
            continue
        whole = b"".join(oracle.pack_scalar(FMT_W6E3M2_P24, np.array([codes[32 * i:32 * i + 32]])).tobytes()
                         for i in range(2))
        assert whole != expected and len(whole) == len(expected)
