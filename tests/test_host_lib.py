"""CPU tests of libwq's host half: exported symbols, sizes, quantize+pack bit-identical to the oracle,
unpack round trips and every synchronous error path. No GPU calls."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from weight_only_quantized_dequant_amd import wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(wq.LIB_PATH), reason="libwq.so not built")


def declared_functions():
    import glob
    src = "".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "wq_linear" in names and "wq_pack_fp6" in names and len(names) >= 12
    L = wq.lib()
    for name in names:
        assert hasattr(L, name), name


def test_read_probe_library_rejects_bad_arguments_before_any_launch():
    # the plain-read probe that bench.py times beside the linears: built with libwq, and every
    # argument error returns -1 without touching the device
    path = os.path.join(os.path.dirname(wq.LIB_PATH), "libwq_probe.so")
    assert os.path.exists(path)
    P = ctypes.CDLL(path)
    f = P.wq_probe_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    a = 1 << 20   # an aligned address the checks stop before any use
    assert f(None, 1024, 4096, 2, a, 1024, None) == -1                 # no buffer
    assert f(a, 1024, 4096, 2, None, 1024, None) == -1                 # no sink
    assert f(a, 1000, 4096, 2, a, 1024, None) == -1                    # not a multiple of 16 bytes
    assert f(a, 1024, 4098, 2, a, 1024, None) == -1                    # waves not a multiple of 4
    assert f(a, 1024, 8192, 2, a, 1024, None) == -1                    # sink smaller than waves / 4 words
    assert f(a, 1024, 4096, 3, a, 1024, None) == -1                    # 2 or 4 loads in flight only
    assert f(a + 8, 1024, 4096, 2, a, 1024, None) == -1                # buffer not 16-byte aligned
    e = P.wq_probe_empty
    e.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    e.restype = ctypes.c_int
    assert e(1, None, None) == -1 and e(0, a, None) == -1              # no sink; no workgroups


def test_version_and_status_strings():
    assert wq.wq_version() >> 16 == 1
    for s in range(-8, 1):
        assert wq.wq_status_string(s) and wq.wq_status_string(s) != "unknown status"
    # no launch has failed on this thread (none ran): no device error to name
    assert wq.wq_last_device_error() == "none"


@pytest.mark.parametrize("fmt", [wq.FMT_F16, wq.FMT_W8, wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1, wq.FMT_BF16,
                                 wq.FMT_W5E2M2, wq.FMT_W3G32, wq.FMT_W6E3M2_P24])
@pytest.mark.parametrize("n,k", [(1, 32), (7, 64), (33, 96), (4096, 11008)])
def test_sizes_match_oracle(fmt, n, k):
    assert wq.wq_packed_bytes(fmt, n, k) == oracle.packed_bytes(fmt, n, k)
    assert wq.wq_scales_bytes(fmt, n, k) == 2 * oracle.scales_count(fmt, n, k)
    assert wq.wq_zeros_bytes(fmt, n, k) == 2 * oracle.zeros_count(fmt, n, k)
    # the size calls ignore the activation flag
    assert wq.wq_packed_bytes(fmt | wq.ACT_BF16, n, k) == oracle.packed_bytes(fmt, n, k)
    assert wq.wq_scales_bytes(fmt | wq.ACT_BF16, n, k) == 2 * oracle.scales_count(fmt, n, k)
    assert wq.wq_zeros_bytes(fmt | wq.ACT_BF16, n, k) == 2 * oracle.zeros_count(fmt, n, k)


def test_sizes_reject_bad_shapes():
    assert wq.wq_packed_bytes(wq.FMT_W8 | 0x200, 4, 64) == 0
    for fmt in range(9):
        assert wq.wq_packed_bytes(fmt, 4, 48) == 0
        assert wq.wq_packed_bytes(fmt, 0, 64) == 0
        assert wq.wq_packed_bytes(fmt, 4, 0) == 0
    assert wq.wq_packed_bytes(9, 4, 64) == 0


def _adversarial(n, k, seed):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    if n >= 8:
        w[0, :] = 0.0
        w[1, 3] = 3.0
        w[2, :] = np.abs(w[2, :])
        w[3, :] = -np.abs(w[3, :])
        w[4, :32] = 1e-9
        w[5, 7] = -0.0
        w[6, :] *= 1e-5
        w[7, :32] = np.linspace(-1, 1, 32, dtype=np.float32)
    return w


def _exact_ties(fmt):
    """Rows whose quotients w/s land exactly on rounding midpoints (scale 1 or 2^k)."""
    rows = []
    if fmt == wq.FMT_W8:
        r = np.zeros(64, dtype=np.float32); r[0] = 127.0; r[1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5]
        rows.append(r)
    if fmt in (wq.FMT_W6E3M2, wq.FMT_W6E3M2_P24):
        r = np.zeros(64, dtype=np.float32); r[0] = 28.0
        r[1:12] = [1.875, 0.03125, 0.09375, 26.0, -26.0, 5.5, -0.0, -0.01, 3.25, 0.40625, 14.999]
        rows.append(r)
    if fmt == wq.FMT_W4E2M1:
        # s = 1: midpoints between neighbouring e2m1 values, both signs, and past-max values
        r = np.zeros(64, dtype=np.float32); r[0] = 6.0
        r[1:14] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -1.75, -5.0, -0.0, 0.2499, 5.0001]
        rows.append(r)
    if fmt == wq.FMT_W5E2M2:
        # s = 1: midpoints between neighbouring e2m2 values, both signs, and past-max values
        r = np.zeros(64, dtype=np.float32); r[0] = 7.0
        r[1:17] = [0.125, 0.375, 0.625, 1.125, 1.875, 2.25, 3.75, 4.5, 6.5, -0.125, -1.375, -6.5, -0.0, 0.1249, 6.5001,
                   -7.25]
        rows.append(r)
    if fmt == wq.FMT_W4G32:
        r = np.zeros(64, dtype=np.float32); r[0] = -7.5; r[1] = 7.5; r[2:6] = [0.5, 1.5, -0.5, 2.5]   # s = 1, z = 8 (7.5 -> even)
        rows.append(r)
    if fmt == wq.FMT_W3G32:
        r = np.zeros(64, dtype=np.float32); r[0] = -3.5; r[1] = 3.5; r[2:6] = [0.5, 1.5, -0.5, 2.5]   # s = 1, z = 4 (3.5 -> even)
        r[32] = -2.5; r[33] = 4.5; r[34:37] = [0.5, -1.5, 3.5]                                        # s = 1, z = 2 (2.5 -> even)
        rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("fmt", [wq.FMT_W8, wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1, wq.FMT_W5E2M2, wq.FMT_W3G32,
                                 wq.FMT_W6E3M2_P24])
@pytest.mark.parametrize("n,k,seed", [(8, 64, 0), (9, 96, 1), (33, 128, 2), (300, 4096, 3), (5, 32 * 130, 4)])
def test_pack_bit_identical_to_oracle(fmt, n, k, seed):
    w = _adversarial(n, k, seed)
    packed_o, s_o, z_o, codes_o = oracle.quantize_and_pack(fmt, w)
    if fmt == wq.FMT_W8:
        packed, s = wq.wq_pack_int8(w)
        z = None
    elif fmt == wq.FMT_W4G32:
        packed, s, z = wq.wq_pack_int4(w)
    elif fmt == wq.FMT_W6E3M2:
        packed, s = wq.wq_pack_fp6(w)
        z = None
    elif fmt == wq.FMT_W5E2M2:
        packed, s = wq.wq_pack_fp5(w)
        z = None
    elif fmt == wq.FMT_W3G32:
        packed, s, z = wq.wq_pack_int3(w)
    elif fmt == wq.FMT_W6E3M2_P24:
        packed, s = wq.wq_pack_fp6_p24(w)
        z = None
    else:
        packed, s = wq.wq_pack_fp4(w)
        z = None
    assert np.array_equal(packed, packed_o)
    assert np.array_equal(s, s_o.reshape(-1))
    if fmt in (wq.FMT_W4G32, wq.FMT_W3G32):
        assert np.array_equal(z, z_o.reshape(-1))
    codes, s2, z2 = wq.wq_unpack(fmt, packed, s, z, n, k)
    assert np.array_equal(codes, codes_o)
    assert np.array_equal(s2, s)


@pytest.mark.parametrize("fmt", [wq.FMT_W8, wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1, wq.FMT_W5E2M2, wq.FMT_W3G32,
                                 wq.FMT_W6E3M2_P24])
def test_pack_exact_ties_identical_to_oracle(fmt):
    w = _exact_ties(fmt)
    packed_o, s_o, z_o, _ = oracle.quantize_and_pack(fmt, w)
    fn = {wq.FMT_W8: wq.wq_pack_int8, wq.FMT_W4G32: wq.wq_pack_int4, wq.FMT_W6E3M2: wq.wq_pack_fp6,
          wq.FMT_W4E2M1: wq.wq_pack_fp4, wq.FMT_W5E2M2: wq.wq_pack_fp5, wq.FMT_W3G32: wq.wq_pack_int3,
          wq.FMT_W6E3M2_P24: wq.wq_pack_fp6_p24}[fmt]
    out = fn(w)
    assert np.array_equal(out[0], packed_o)
    assert np.array_equal(out[1], s_o.reshape(-1))
    if fmt in (wq.FMT_W4G32, wq.FMT_W3G32):
        assert np.array_equal(out[2], z_o.reshape(-1))


def test_pack_multithreaded_large_matches_oracle():
    rng = np.random.default_rng(12)
    w = (0.02 * rng.standard_normal((1024, 8192))).astype(np.float32)
    for fmt, fn in ((wq.FMT_W8, wq.wq_pack_int8), (wq.FMT_W4G32, wq.wq_pack_int4)):
        packed_o, s_o, z_o, _ = oracle.quantize_and_pack(fmt, w)
        out = fn(w)
        assert np.array_equal(out[0], packed_o)
        assert np.array_equal(out[1], s_o.reshape(-1))
    # fp6: the oracle's brute-force encoder is slow, so compare a row sample
    packed, s = wq.wq_pack_fp6(w)
    rows = rng.choice(1024, 24, replace=False)
    packed_o, s_o, _, _ = oracle.quantize_and_pack(wq.FMT_W6E3M2, w[rows])
    rb = 8192 * 3 // 4
    got = np.concatenate([packed[r * rb:(r + 1) * rb] for r in rows])
    assert np.array_equal(got, packed_o)
    assert np.array_equal(s[rows], s_o)


def test_unpack_f16_and_round_trip_of_oracle_packing():
    rng = np.random.default_rng(5)
    for fmt, codes in ((wq.FMT_W8, rng.integers(-127, 128, (3, 96)).astype(np.int8)),
                       (wq.FMT_W4G32, rng.integers(0, 16, (3, 96)).astype(np.uint8)),
                       (wq.FMT_W6E3M2, rng.integers(0, 64, (3, 96)).astype(np.uint8)),
                       (wq.FMT_W4E2M1, rng.integers(0, 16, (3, 96)).astype(np.uint8)),
                       (wq.FMT_W5E2M2, rng.integers(0, 32, (3, 96)).astype(np.uint8)),
                       (wq.FMT_F16, rng.integers(0, 65536, (3, 96)).astype(np.uint16))):
        packed = oracle.pack_scalar(fmt, codes)
        got, _, _ = wq.wq_unpack(fmt, packed, np.zeros(9, np.uint16), np.zeros(9, np.uint16), 3, 96)
        assert np.array_equal(got, codes)


def test_scale_rounding_matches_oracle_over_magnitudes():
    # scales span fp16 subnormals, normals and the edge of the range
    mags = np.geomspace(1e-9, 1e6, 400).astype(np.float32)
    w = np.zeros((400, 32), dtype=np.float32)
    w[:, 0] = mags
    w[:, 1] = -mags / 3
    _, s = wq.wq_pack_int8(w)
    _, s_o = oracle.quantize_int8(w)
    assert np.array_equal(s, s_o)
    ok = mags < 1.8e6
    _, s6 = wq.wq_pack_fp6(w[ok & (mags < 1e5)])
    _, s6_o = oracle.quantize_fp6(w[ok & (mags < 1e5)])
    assert np.array_equal(s6, s6_o)


def test_pack_errors():
    w = np.zeros((2, 64), dtype=np.float32)
    L = wq.lib()
    buf = np.zeros(4096, dtype=np.uint8)
    sc = np.zeros(64, dtype=np.uint16)
    p = wq._host_ptr
    assert L.wq_pack_int8(None, 2, 64, p(buf), p(sc)) == -1
    assert L.wq_pack_int8(p(w), 2, 64, None, p(sc)) == -1
    assert L.wq_pack_int4(p(w), 2, 64, p(buf), p(sc), None) == -1
    assert L.wq_pack_int8(p(w), -1, 64, p(buf), p(sc)) == -1
    assert L.wq_pack_int8(p(w), 2, 48, p(buf), p(sc)) == -2
    assert L.wq_pack_fp6(p(w), 0, 64, p(buf), p(sc)) == -2
    assert L.wq_pack_int4(p(w), 2, 0, p(buf), p(sc), p(sc)) == -2
    bad = w.copy()
    bad[1, 5] = np.nan
    with pytest.raises(wq.WqError) as e:
        wq.wq_pack_fp6(bad)
    assert e.value.status == -4
    bad[1, 5] = np.inf
    with pytest.raises(wq.WqError) as e:
        wq.wq_pack_int4(bad)
    assert e.value.status == -4
    big = np.full((1, 32), 1e7, dtype=np.float32)
    with pytest.raises(wq.WqError) as e:
        wq.wq_pack_int8(big)      # 1e7/127 > 65504
    assert e.value.status == -7
    assert L.wq_unpack(9, p(buf), p(sc), p(sc), 2, 64, p(buf), None, None) == -3
    assert L.wq_pack_int3(p(w), 2, 64, p(buf), p(sc), None) == -1
    assert L.wq_pack_int3(p(w), 2, 48, p(buf), p(sc), p(sc)) == -2
    assert L.wq_pack_fp6_p24(p(w), 2, 64, None, p(sc)) == -1
    assert L.wq_pack_fp6_p24(p(w), 0, 64, p(buf), p(sc)) == -2
    with pytest.raises(wq.WqError) as e:
        wq.wq_pack_int3(np.full((1, 32), np.nan, dtype=np.float32))
    assert e.value.status == -4
    with pytest.raises(wq.WqError) as e:
        wq.wq_pack_fp6_p24(np.full((1, 32), 1e7, dtype=np.float32))   # 1e7/28 > 65504
    assert e.value.status == -7
    assert L.wq_pack_fp5(None, 2, 64, p(buf), p(sc)) == -1
    assert L.wq_pack_fp5(p(w), 2, 40, p(buf), p(sc)) == -2
    bad[1, 5] = -np.inf
    with pytest.raises(wq.WqError) as e:
        wq.wq_pack_fp5(bad)
    assert e.value.status == -4
    with pytest.raises(wq.WqError) as e:
        wq.wq_pack_fp5(np.full((1, 32), 1e6, dtype=np.float32))      # 1e6/7 > 65504
    assert e.value.status == -7


def test_device_entry_points_reject_bad_arguments_before_launch():
    # these return before any HIP call, so they run without a GPU
    L = wq.lib()
    a = 1 << 20                                # a 16-byte-aligned fake address, never dereferenced
    assert L.wq_linear(a, a, a, a, a, 1, 64, 64, 9, None) == -3
    assert L.wq_linear(None, a, a, a, a, 1, 64, 64, 1, None) == -1
    assert L.wq_linear(a, a, None, None, a, 1, 64, 64, 1, None) == -1
    assert L.wq_linear(a, a, a, None, a, 1, 64, 64, 2, None) == -1
    assert L.wq_linear(a, a, a, a, a, 0, 64, 64, 1, None) == -2
    assert L.wq_linear(a, a, a, a, a, 1, 64, 48, 1, None) == -2
    assert L.wq_linear(a, a, a, a, a, 1, 0, 64, 1, None) == -2
    assert L.wq_linear(a + 8, a, a, a, a, 1, 64, 64, 1, None) == -5
    assert L.wq_linear(a, a, a, a, a + 2, 1, 64, 64, 1, None) == -5
    assert L.wq_dequant(1, a, a, a, a, 64, 40, None) == -2
    assert L.wq_dequant(5, a, a, a, a, 64, 64, None) == -3
    # the activation flag: bfloat16 x with fp16 weights, fp16 x with bfloat16 weights and unknown
    # flags are format errors; a bfloat16 code otherwise passes the same checks
    assert L.wq_linear(a, a, a, a, a, 1, 64, 64, wq.FMT_F16 | wq.ACT_BF16, None) == -3
    assert L.wq_linear(a, a, a, a, a, 1, 64, 64, wq.FMT_BF16, None) == -3
    assert L.wq_linear(a, a, a, a, a, 1, 64, 64, wq.FMT_W8 | 0x200, None) == -3
    assert L.wq_dequant(wq.FMT_F16 | wq.ACT_BF16, a, a, a, a, 64, 64, None) == -3
    assert L.wq_linear(a, a, a, None, a, 1, 64, 64, wq.FMT_W4G32 | wq.ACT_BF16, None) == -1
    assert L.wq_linear(a, a, None, None, a, 1, 64, 64, wq.FMT_W8 | wq.ACT_BF16, None) == -1
    assert L.wq_linear(a, a, a, a, a, 1, 64, 48, wq.FMT_BF16 | wq.ACT_BF16, None) == -2
    assert L.wq_linear(a + 8, a, a, a, a, 1, 64, 64, wq.FMT_W6E3M2 | wq.ACT_BF16, None) == -5
    assert L.wq_dequant(2, a, a, None, a, 64, 64, None) == -1
    assert L.wq_dequant(1, a + 4, a, a, a, 64, 64, None) == -5
    assert L.wq_linear(a, a, a, a, a, 1, 64, (1 << 26) + 32, 1, None) == -2    # K above 2^26
    assert L.wq_linear(a, a, a, a, a, 1, 1 << 22, 1 << 20, 1, None) == -2       # N*K/32 above int32
    assert wq.wq_linear_kernel_name(2, 1, 4096, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(3, 16, 4096, 4096) == "lm_kernel<3, 1, 1>"
    assert wq.wq_linear_kernel_name(3, 16, 8192, 4096) == "lm_kernel<3, 2, 1>"
    assert wq.wq_linear_kernel_name(1, 16, 4096, 4096).startswith("mfma_kernel")
    assert wq.wq_linear_kernel_name(0, 16, 4096, 4096).startswith("mfma_kernel")
    # W4 on the matrix cores: through LDS when K is a multiple of 256, else fragment loads
    assert wq.wq_linear_kernel_name(2, 8, 4096, 4096) == "lm_kernel<2, 1, 1>"
    assert wq.wq_linear_kernel_name(2, 8, 4096, 4128) == "mfma_kernel<2, 1>"
    # M = 2 and 3: the LDS-staged kernel on large matrices (N*K >= 2^24) from 3 rows, from 2 for FP4
    # and FP5; the GEMV below that, for W8, and for W4 / int3 with K not a multiple of 256
    assert wq.wq_linear_kernel_name(3, 3, 4096, 4096) == "lm_kernel<3, 1, 1>"
    assert wq.wq_linear_kernel_name(3, 3, 2048, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(3, 2, 4096, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(2, 3, 4096, 4096) == "lm_kernel<2, 1, 1>"
    assert wq.wq_linear_kernel_name(2, 2, 4096, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(2, 3, 4096, 4128).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(7, 3, 11008, 4096) == "lm_kernel<7, 2, 1>"
    assert wq.wq_linear_kernel_name(4, 2, 4096, 4096) == "lm_kernel<4, 1, 1>"
    assert wq.wq_linear_kernel_name(6, 2, 4096, 4096) == "lm_kernel<6, 1, 1>"
    assert wq.wq_linear_kernel_name(4, 1, 4096, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(1, 3, 11008, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_grouped_kernel_name(2, 3, [(4096, 4096), (11008, 4096), (4096, 11008)]) == \
        "lm_grouped_kernel<2, 2, 1>"
    # bfloat16 x: W6 from 3 rows as with fp16 x, W4 on the GEMV up to 3 rows
    assert wq.wq_linear_kernel_name(3 | wq.ACT_BF16, 3, 4096, 4096) == "lm_kernel<259, 1, 1>"
    assert wq.wq_linear_kernel_name(2 | wq.ACT_BF16, 3, 4096, 4096).startswith("gemv_kernel<258, 3,")
    assert wq.wq_linear_kernel_name(2 | wq.ACT_BF16, 4, 4096, 4096) == "lm_kernel<258, 1, 1>"
    assert wq.wq_linear_grouped_kernel_name(2 | wq.ACT_BF16, 3, [(4096, 4096), (11008, 4096)]).startswith(
        "gemv_grouped_kernel<258, 3,")
    # M = 4: the matrix cores for W6 with N >= 2048, W8 with N >= 4096 and W4 from N*K = 2^24, the GEMV otherwise
    assert wq.wq_linear_kernel_name(3, 4, 4096, 4096).startswith("lm_kernel")
    assert wq.wq_linear_kernel_name(3, 4, 2048, 4096).startswith("lm_kernel")
    assert wq.wq_linear_kernel_name(1, 4, 8192, 4096).startswith("mfma_kernel")
    assert wq.wq_linear_kernel_name(1, 4, 2048, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(3, 4, 1280, 8192).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(2, 4, 2048, 4096).startswith("gemv_kernel")
    assert wq.wq_linear_kernel_name(2, 4, 4096, 4096) == "lm_kernel<2, 1, 1>"
    assert wq.wq_linear_kernel_name(2, 4, 8192, 8192) == "lm_kernel<2, 2, 1>"
    assert wq.wq_linear_kernel_name(3, 16, 4096, 40) == ""
    # grouped: the GEMV takes its rows per wave from the largest item
    assert wq.wq_linear_grouped_kernel_name(3, 1, [(8192, 8192), (1024, 8192)]) == "gemv_grouped_kernel<3, 1, 4>"
    # ... and the matrix-core kernels take their family and row blocks from it too
    assert wq.wq_linear_grouped_kernel_name(3, 8, [(1024, 8192), (8192, 8192)]) == "lm_grouped_kernel<3, 2, 1>"
    assert wq.wq_linear_grouped_kernel_name(2, 4, [(8192, 8192), (1024, 8192)]) == "lm_grouped_kernel<2, 2, 1>"
    assert wq.wq_linear_grouped_kernel_name(2, 8, [(8192, 8192), (1024, 8224)]) == "mfma_grouped_kernel<2, 1>"
    assert wq.wq_linear_grouped_kernel_name(1, 16, [(4096, 4096), (16384, 4096)]) == "mfma_grouped_kernel<1, 4>"
    # 17..64 rows of x: the LDS-staged kernel takes 2 or 4 tiles of 16 rows in one launch
    # (W4 when K is a multiple of 256); the others, and more than 64 rows, run in slabs
    assert wq.wq_linear_kernel_name(3, 20, 8192, 8192) == "lm_kernel<3, 2, 2>"
    assert wq.wq_linear_kernel_name(2, 64, 4096, 4096) == "lm_kernel<2, 1, 4>"
    assert wq.wq_linear_kernel_name(2, 64, 4096, 4128) == "mfma_kernel<2, 1>"
    assert wq.wq_linear_kernel_name(1, 40, 4096, 4096) == "mfma_kernel<1, 1>"
    # W8 and fp16 weights (decode launches of 16 rows each) from 17 rows: the tiled kernel when
    # its chain of K steps costs less than the 16-row launches' weight streams
    assert wq.wq_linear_kernel_name(1, 17, 11008, 4096) == "mfma_kernel<1, 2>"
    assert wq.wq_linear_kernel_name(1, 33, 11008, 4096) == "pf_kernel<1>"
    assert wq.wq_linear_kernel_name(0, 17, 11008, 4096) == "pf_kernel<0>"
    assert wq.wq_linear_kernel_name(0, 16, 11008, 4096) == "mfma_kernel<0, 2>"
    assert wq.wq_linear_kernel_name(0, 17, 4096, 4096) == "mfma_kernel<0, 1>"
    assert wq.wq_linear_kernel_name(0, 65, 4096, 4096) == "pf_kernel<0>"
    assert wq.wq_linear_kernel_name(0, 40, 4096, 11008) == "mfma_kernel<0, 1>"   # 172 steps, 32 tiles
    # 65..192 rows: the tiled prefill kernel when the linear has enough 128 x 128 tiles for its
    # chain of K steps (K / 64 at most 2x the tiles for W4, 4x for W8/W6/FP4, any for fp16
    # weights); else 64-row launches
    assert wq.wq_linear_kernel_name(3, 100, 4096, 4096) == "pf_kernel<3>"      # 64 steps, 32 tiles
    assert wq.wq_linear_kernel_name(2, 100, 4096, 4096) == "pf_kernel<2>"
    assert wq.wq_linear_kernel_name(2, 100, 4096, 8192) == "lm_kernel<2, 1, 4>"   # 128 steps
    assert wq.wq_linear_kernel_name(2, 129, 4096, 8192) == "pf_kernel<2>"      # 64 tiles
    assert wq.wq_linear_kernel_name(3, 128, 4096, 11008) == "lm_kernel<3, 1, 4>"   # 172 steps, 32 tiles
    assert wq.wq_linear_kernel_name(3, 160, 4096, 11008) == "pf_kernel<3>"     # 64 tiles
    assert wq.wq_linear_kernel_name(2, 192, 8192, 28672) == "lm_kernel<2, 2, 4>"   # 448 steps, 128 tiles
    assert wq.wq_linear_kernel_name(0, 65, 4096, 11008) == "pf_kernel<0>"
    assert wq.wq_linear_kernel_name(3, 64, 4096, 4096) == "lm_kernel<3, 1, 4>"
    # from 193 rows of x on: the tiled prefill kernel always, one launch for all rows
    assert wq.wq_linear_kernel_name(2, 192, 4096, 11008) == "lm_kernel<2, 1, 4>"
    assert wq.wq_linear_kernel_name(2, 193, 4096, 11008) == "pf_kernel<2>"
    assert wq.wq_linear_kernel_name(3, 193, 4096, 4096) == "pf_kernel<3>"
    assert wq.wq_linear_kernel_name(2, 600, 4096, 4128) == "pf_kernel<2>"
    assert wq.wq_linear_kernel_name(2 | wq.ACT_BF16, 512, 11008, 4096) == "pf_kernel<258>"
    assert wq.wq_linear_kernel_name(0, 4096, 4096, 4096) == "pf_kernel<0>"
    # rows of 2^25 + 256 and more: 16-row slabs (32-bit x offsets stay in range)
    assert wq.wq_linear_kernel_name(3, 64, 64, (1 << 25) + 256) == "lm_kernel<3, 1, 1>"
    assert wq.wq_linear_kernel_name(3, 64, 64, 1 << 25) == "lm_kernel<3, 1, 4>"
    assert wq.wq_linear_grouped_kernel_name(3, 40, [(64, 4096), (64, (1 << 25) + 256)]) == "lm_kernel<3, 1, 1>"
    assert wq.wq_linear_grouped_kernel_name(3, 16, [(64, 4096), (64, (1 << 25) + 256)]) == "lm_grouped_kernel<3, 1, 1>"
    assert wq.wq_linear_grouped_kernel_name(3, 20, [(1024, 8192), (8192, 8192)]) == "lm_grouped_kernel<3, 2, 2>"
    assert wq.wq_linear_grouped_kernel_name(3, 65, [(1024, 8192), (8192, 8192)]) == "pf_grouped_kernel<3>"
    # a group whose longest chain is too long for its tiles: one call per item (the largest shown)
    assert wq.wq_linear_grouped_kernel_name(3, 65, [(1024, 28672), (8192, 8192)]) == "pf_kernel<3>"
    assert wq.wq_linear_grouped_kernel_name(3, 65, [(1024, 28672), (1024, 8192)]) == "lm_kernel<3, 1, 4>"
    # prefill-sized M: the tiles of every item in one launch (one item: the plain tiled kernel)
    assert wq.wq_linear_grouped_kernel_name(3, 512, [(1024, 8192), (8192, 8192)]) == "pf_grouped_kernel<3>"
    assert wq.wq_linear_grouped_kernel_name(2 | wq.ACT_BF16, 193, [(4096, 4096)] * 3) == "pf_grouped_kernel<258>"
    assert wq.wq_linear_grouped_kernel_name(3, 512, [(8192, 28672)]) == "pf_kernel<3>"
    assert wq.wq_linear_grouped_kernel_name(3, 192, [(1024, 8192), (8192, 8192)]) == "pf_grouped_kernel<3>"
    assert wq.wq_linear_grouped_kernel_name(2, 100, [(1024, 8192), (8192, 8192)]) == "pf_grouped_kernel<2>"
    assert wq.wq_linear_grouped_kernel_name(2, 100, [(1024, 8192), (1024, 8192)]) == "lm_kernel<2, 1, 4>"
    assert wq.wq_linear_grouped_kernel_name(2, 100, [(4096, 4096)] * 3) == "pf_grouped_kernel<2>"
    assert wq.wq_linear_grouped_kernel_name(1, 20, [(1024, 8192), (8192, 8192)]) == "mfma_kernel<1, 2>"
    # the LDS-staged group takes two row blocks per wave when any item has 8192 rows or more,
    # whatever the order of equal-size items
    assert wq.wq_linear_grouped_kernel_name(2, 16, [(4096, 11008), (11008, 4096)]) == "lm_grouped_kernel<2, 2, 1>"
    assert wq.wq_linear_grouped_kernel_name(2, 16, [(11008, 4096), (4096, 11008)]) == "lm_grouped_kernel<2, 2, 1>"
    assert wq.wq_linear_grouped_kernel_name(3, 16, [(3584, 8192), (8192, 3584), (1280, 8192)]) == "lm_grouped_kernel<3, 2, 1>"
    # FP4: the GEMV up to M = 3 (and M = 4 below N*K = 2^24), the LDS-staged kernel above, for any K
    assert wq.wq_linear_kernel_name(4, 1, 4096, 4096) == "gemv_kernel<4, 1, 4>"
    assert wq.wq_linear_kernel_name(4, 4, 2048, 4096) == "gemv_kernel<4, 4, 4>"
    assert wq.wq_linear_kernel_name(4, 4, 4096, 4096) == "lm_kernel<4, 1, 1>"
    assert wq.wq_linear_kernel_name(4, 8, 4096, 4128) == "lm_kernel<4, 1, 1>"
    assert wq.wq_linear_kernel_name(4, 16, 8192, 4096) == "lm_kernel<4, 2, 1>"
    assert wq.wq_linear_kernel_name(4, 64, 4096, 4096) == "lm_kernel<4, 1, 4>"
    assert wq.wq_linear_kernel_name(4, 100, 4096, 4096) == "pf_kernel<4>"
    assert wq.wq_linear_kernel_name(4, 100, 4096, 11008) == "lm_kernel<4, 1, 4>"
    assert wq.wq_linear_grouped_kernel_name(4, 1, [(4096, 4096), (11008, 4096)]) == "gemv_grouped_kernel<4, 1, 4>"
    assert wq.wq_linear_grouped_kernel_name(4, 8, [(1024, 8192), (8192, 8224)]) == "lm_grouped_kernel<4, 2, 1>"
    # bfloat16 activations: the same plan, named with the combined code (format | 0x100)
    bf = wq.ACT_BF16
    assert wq.wq_linear_kernel_name(2 | bf, 1, 4096, 4096) == "gemv_kernel<258, 1, 4>"
    assert wq.wq_linear_kernel_name(2 | bf, 8, 4096, 4096) == "lm_kernel<258, 1, 1>"
    assert wq.wq_linear_kernel_name(2 | bf, 8, 4096, 4128) == "mfma_kernel<258, 1>"
    assert wq.wq_linear_kernel_name(3 | bf, 16, 8192, 4096) == "lm_kernel<259, 2, 1>"
    assert wq.wq_linear_kernel_name(1 | bf, 16, 4096, 4096) == "mfma_kernel<257, 1>"
    assert wq.wq_linear_kernel_name(5 | bf, 1, 16384, 4096) == "gemv_kernel<261, 1, 1>"
    assert wq.wq_linear_kernel_name(5 | bf, 16, 8192, 4096) == "mfma_kernel<261, 2>"
    assert wq.wq_linear_kernel_name(4 | bf, 64, 4096, 4096) == "lm_kernel<260, 1, 4>"
    assert wq.wq_linear_kernel_name(0 | bf, 1, 4096, 4096) == ""
    assert wq.wq_linear_kernel_name(5, 1, 4096, 4096) == ""
    assert wq.wq_linear_grouped_kernel_name(2 | bf, 1, [(4096, 4096), (11008, 4096)]) == "gemv_grouped_kernel<258, 1, 4>"


def test_kernel_name_thresholds_stated_in_the_header():
    # include/wq.h: the decode kernels take up to 64 rows of x per launch for W6, FP4, FP5 and W4
    # with K a multiple of 256 (16 otherwise); the tiled kernel takes all rows from 193 on, and from
    # 17 (W8, fp16 weights), 65 (W4, W6, FP4) or 81 (FP5) rows where its chain is short enough
    big = (4096, 4096)                                  # 64 K steps, 32 tiles of 128 weight rows
    for fmt in (wq.FMT_W8, wq.FMT_F16):
        assert wq.wq_linear_kernel_name(fmt, 16, *big).startswith("mfma_kernel")
        assert not wq.wq_linear_kernel_name(fmt, 16, 11008, 4096).startswith("pf_kernel")
        assert wq.wq_linear_kernel_name(fmt, 40, 11008, 4096) == "pf_kernel<%d>" % fmt
    for fmt in (wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1):
        assert wq.wq_linear_kernel_name(fmt, 64, *big) == "lm_kernel<%d, 1, 4>" % fmt
        assert wq.wq_linear_kernel_name(fmt, 65, *big) == "pf_kernel<%d>" % fmt
    for fmt in (wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1, wq.FMT_W5E2M2, wq.FMT_W8, wq.FMT_F16):
        assert wq.wq_linear_kernel_name(fmt, 193, 4096, 28672) == "pf_kernel<%d>" % fmt
    for fmt in (wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1, wq.FMT_W5E2M2):   # 448 K steps, 64 tiles
        assert wq.wq_linear_kernel_name(fmt, 192, 4096, 28672) == "lm_kernel<%d, 1, 4>" % fmt


def test_fp5_kernel_choice():
    # FP5 e2m2: the VALU GEMV at M = 1, and up to M = 4 below N*K = 2^24; the LDS-staged kernel from
    # M = 2 above that and from M = 5 always (1 to 4 tiles of 16 rows), the tiled kernel from 81 rows
    # when its chain is short enough
    f = wq.FMT_W5E2M2
    assert wq.wq_linear_kernel_name(f, 1, 4096, 4096) == "gemv_kernel<6, 1, 4>"
    assert wq.wq_linear_kernel_name(f, 3, 4096, 4096) == "lm_kernel<6, 1, 1>"
    assert wq.wq_linear_kernel_name(f, 3, 2048, 4096) == "gemv_kernel<6, 3, 4>"
    assert wq.wq_linear_kernel_name(f, 4, 2048, 4096) == "gemv_kernel<6, 4, 4>"
    assert wq.wq_linear_kernel_name(f, 4, 4096, 4096) == "lm_kernel<6, 1, 1>"
    assert wq.wq_linear_kernel_name(f, 5, 2048, 4096) == "lm_kernel<6, 1, 1>"
    assert wq.wq_linear_kernel_name(f, 5, 8192, 8192) == "lm_kernel<6, 2, 1>"
    assert wq.wq_linear_kernel_name(f, 17, 4096, 4096) == "lm_kernel<6, 1, 2>"
    assert wq.wq_linear_kernel_name(f, 64, 4096, 4096) == "lm_kernel<6, 1, 4>"
    assert wq.wq_linear_kernel_name(f, 65, 4096, 4096) == "lm_kernel<6, 1, 4>"
    assert wq.wq_linear_kernel_name(f, 80, 4096, 4096) == "lm_kernel<6, 1, 4>"
    assert wq.wq_linear_kernel_name(f, 81, 4096, 4096) == "pf_kernel<6>"
    assert wq.wq_linear_kernel_name(f | wq.ACT_BF16, 81, 4096, 4096) == "pf_kernel<262>"
    assert wq.wq_linear_grouped_kernel_name(f, 8, [(4096, 4096), (11008, 4096)]) == "lm_grouped_kernel<6, 2, 1>"
    assert wq.wq_linear_grouped_kernel_name(f, 1, [(4096, 4096), (11008, 4096)]) == "gemv_grouped_kernel<6, 1, 4>"


def test_linear_silu_rejects_bad_arguments_before_launch():
    L = wq.lib()
    a = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails its checks first
    assert L.wq_linear_silu(a, a, a, a, a, 1, 64, 256, wq.FMT_W8 | wq.ACT_BF16, None) == -3
    assert L.wq_linear_silu(a, a, a, a, a, 1, 64, 256, 9, None) == -3
    assert L.wq_linear_silu(a, a, a, a, a, 1, 0, 256, wq.FMT_W8, None) == -2
    assert L.wq_linear_silu(a, a, a, a, a, 1, -1, 256, wq.FMT_W8, None) == -1
    assert L.wq_linear_silu(a, a, a, a, a, 1, 64, 48, wq.FMT_W8, None) == -2
    assert L.wq_linear_silu(a, a, a, None, a, 1, 64, 256, wq.FMT_W4G32, None) == -1   # W4 needs zeros
    assert L.wq_linear_silu(a, a, a, a, ctypes.c_void_p((1 << 20) + 2), 1, 64, 256, wq.FMT_W8, None) == -5


def test_int3_and_split_fp6_kernel_choice():
    # int3 follows W4's plan (groups of 32: the LDS-staged kernel needs K a multiple of 256, else
    # the fragment-load kernel), the 2+4 FP6 layout follows W6's (same slices, other decode);
    # neither takes bfloat16 activations
    f3, f6 = wq.FMT_W3G32, wq.FMT_W6E3M2_P24
    assert wq.wq_linear_kernel_name(f3, 1, 4096, 4096) == "gemv_kernel<7, 1, 4>"
    assert wq.wq_linear_kernel_name(f3, 4, 2048, 4096) == "gemv_kernel<7, 4, 4>"
    assert wq.wq_linear_kernel_name(f3, 4, 4096, 4096) == "lm_kernel<7, 1, 1>"
    assert wq.wq_linear_kernel_name(f3, 8, 8192, 8192) == "lm_kernel<7, 2, 1>"
    assert wq.wq_linear_kernel_name(f3, 8, 4096, 4096 + 32) == "mfma_kernel<7, 1>"
    assert wq.wq_linear_kernel_name(f3, 64, 4096, 4096) == "lm_kernel<7, 1, 4>"
    assert wq.wq_linear_kernel_name(f3, 65, 4096, 4096) == "pf_kernel<7>"
    for m, n, k in ((1, 4096, 4096), (4, 2048, 4096), (4, 4096, 4096), (8, 28672, 8192), (16, 8192, 8192),
                    (64, 4096, 4096), (65, 4096, 4096), (193, 4096, 28672)):
        want = wq.wq_linear_kernel_name(wq.FMT_W6E3M2, m, n, k).replace("<3", "<8")
        assert wq.wq_linear_kernel_name(f6, m, n, k) == want, (m, n, k)
    assert wq.wq_linear_grouped_kernel_name(f3, 8, [(4096, 4096), (11008, 4096)]) == "lm_grouped_kernel<7, 2, 1>"
    assert wq.wq_linear_grouped_kernel_name(f3, 8, [(4096, 4096), (4096, 4128)]) == "mfma_grouped_kernel<7, 1>"
    assert wq.wq_linear_grouped_kernel_name(f6, 1, [(10240, 8192), (8192, 8192)]) == "gemv_grouped_kernel<8, 1, 4>"
    for f in (f3, f6):
        assert wq.wq_linear_kernel_name(f | wq.ACT_BF16, 1, 4096, 4096) == ""


class _FakeDeviceTensor:
    """Looks like a contiguous GPU tensor of `nbytes` bytes to the binding's checks; never launched."""

    is_cuda = True

    def __init__(self, nbytes, contiguous=True):
        self.nbytes, self.contiguous = nbytes, contiguous

    def get_device(self):
        return 0

    def is_contiguous(self):
        return self.contiguous

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1

    def data_ptr(self):
        return 1 << 20


def test_binding_rejects_cpu_strided_and_short_buffers_before_any_launch(monkeypatch):
    import torch
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    m, n, k, fmt = 2, 64, 256, wq.FMT_W4G32
    good = dict(x=_FakeDeviceTensor(2 * m * k), w=_FakeDeviceTensor(wq.wq_packed_bytes(fmt, n, k)),
                s=_FakeDeviceTensor(wq.wq_scales_bytes(fmt, n, k)), z=_FakeDeviceTensor(wq.wq_zeros_bytes(fmt, n, k)),
                y=_FakeDeviceTensor(2 * m * n))

    def call(**over):
        a = dict(good, **over)
        wq.wq_linear(a["x"], a["w"], a["s"], a["z"], a["y"], m, n, k, fmt)

    cpu = torch.zeros(4096, dtype=torch.int16)
    for name in ("x", "w", "s", "z", "y"):
        with pytest.raises(ValueError, match="GPU tensor"):
            call(**{name: cpu})
        with pytest.raises(ValueError, match="bytes"):
            call(**{name: _FakeDeviceTensor(good[name].nbytes - 1)})
        with pytest.raises(ValueError, match="contiguous"):
            call(**{name: _FakeDeviceTensor(good[name].nbytes, contiguous=False)})
    with pytest.raises(ValueError, match="item 1"):
        wq.wq_linear_grouped([(good["x"], good["w"], good["s"], good["z"], good["y"], n, k),
                              (good["x"], good["w"], good["s"], good["z"], _FakeDeviceTensor(2 * m * n - 2), n, k)],
                             m, fmt)
    with pytest.raises(ValueError, match="w_out"):
        wq.wq_dequant(fmt, good["w"], good["s"], good["z"], _FakeDeviceTensor(2 * n * k - 1), n, k)
    with pytest.raises(ValueError, match="packed"):
        wq.wq_dequant(fmt, cpu, good["s"], good["z"], _FakeDeviceTensor(2 * n * k), n, k)
    # the bf16 flag changes no size: a short y is short for either activation type
    with pytest.raises(ValueError, match="y holds"):
        wq.wq_linear(good["x"], good["w"], good["s"], good["z"], _FakeDeviceTensor(2 * m * n - 1), m, n, k,
                     fmt | wq.ACT_BF16)


def test_rope_table_matches_the_oracle_angles():
    from oracle import decode as D
    cos, sin = wq.wq_rope_table(10000.0, 128, 300)
    for p in (0, 1, 17, 299):
        a = D.rope_angles(p, 128, 10000.0)
        assert np.allclose(cos[p], np.cos(a), rtol=0, atol=6e-8)   # float32 rounding of the float64 value
        assert np.allclose(sin[p], np.sin(a), rtol=0, atol=6e-8)
    assert np.array_equal(cos[0], np.ones(64, dtype=np.float32)) and not np.any(sin[0])
    L = wq.lib()
    buf = np.zeros(64, dtype=np.float32)
    assert L.wq_rope_table(10000.0, 3, 4, wq._host_ptr(buf), wq._host_ptr(buf)) == -2
    assert L.wq_rope_table(-1.0, 4, 4, wq._host_ptr(buf), wq._host_ptr(buf)) == -1


def test_decode_entry_points_reject_bad_arguments_before_launch():
    L = wq.lib()
    a = 1 << 20
    assert L.wq_embed(a, a, a, 1, 12, 10, None) == -2                 # d not a multiple of 8
    assert L.wq_embed(None, a, a, 1, 16, 10, None) == -1
    assert L.wq_add_rmsnorm(a, None, a, -1.0, a, 1, 16, None) == -1   # eps < 0
    assert L.wq_add_rmsnorm(a + 4, None, a, 1e-5, a, 1, 16, None) == -5
    assert L.wq_silu_mul(a, a, a, 0, None) == -2
    assert L.wq_argmax_next(a, 0, 16, a, a, None) == -2
    assert L.wq_rope_attention(a, a, a, a, a, a, a, a, a, 1, 6, 4, 128, 16, None, 0, None) == -2   # 6 % 4
    assert L.wq_rope_attention(a, a, a, a, a, a, a, a, a, 1, 4, 4, 128, 5000, None, 0, None) == -1  # no workspace
    need = wq.wq_attention_workspace_bytes(1, 4, 128, 5000)
    # caches of up to 4096 positions take one workgroup per head and no workspace; longer ones the chunks
    assert need > 0 and wq.wq_attention_workspace_bytes(1, 4, 128, 4096) == 0 and wq.wq_attention_workspace_bytes(1, 4, 128, 4097) > 0
    assert L.wq_rope_attention(a, a, a, a, a, a, a, a, a, 1, 4, 4, 128, 5000, a, need - 1, None) == -1


def test_decode_binding_rejects_cpu_and_short_buffers(monkeypatch):
    import torch
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    F = _FakeDeviceTensor
    with pytest.raises(ValueError, match="x holds"):
        wq.wq_add_rmsnorm(F(4 * 2 * 64 - 4), None, F(128), 1e-5, F(256), 2, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        wq.wq_silu_mul(torch.zeros(64, dtype=torch.int16), F(128), F(128), 64)
    with pytest.raises(ValueError, match="cache_v"):
        m, H, Hkv, hd, S = 1, 4, 2, 64, 16
        wq.wq_rope_attention(F(2 * H * hd), F(2 * Hkv * hd), F(2 * Hkv * hd), F(2 * S * Hkv * hd),
                             F(2 * S * Hkv * hd - 2), F(4 * S * hd // 2), F(4 * S * hd // 2), F(4), F(2 * H * hd),
                             m, H, Hkv, hd, S, None)
    with pytest.raises(ValueError, match="workspace"):
        m, H, Hkv, hd, S = 1, 4, 2, 64, 4160
        need = wq.wq_attention_workspace_bytes(m, H, hd, S)
        wq.wq_rope_attention(F(2 * H * hd), F(2 * Hkv * hd), F(2 * Hkv * hd), F(2 * S * Hkv * hd),
                             F(2 * S * Hkv * hd), F(4 * S * hd // 2), F(4 * S * hd // 2), F(4), F(2 * H * hd),
                             m, H, Hkv, hd, S, F(need - 1))
