"""GPU parity: libwq's device path (through the C ABI) against the CPU oracle.

* wq_dequant: bit-exact fp16 patterns (+-0 included) for every format.
* wq_linear: within the oracle's closed-form error bound and rtol = atol = 1e-2, for
  every M in 1..16 (and slabs above 16), ragged N and K, one-hot x bit-exact, x = 0
  exact, and repeat calls bit-identical.
* The workloads at full size, in the launch configuration the benchmark times, on
  sampled output rows that the oracle computes row by row.
"""

import numpy as np
import pytest

import oracle
from weight_only_quantized_dequant_amd import inputs, wq
from tests.gpu_util import DeviceWeights, check_linear, dev, host_bits, oracle_rows, torch_cuda

pytestmark = pytest.mark.gpu

FMTS = [wq.FMT_W8, wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1, wq.FMT_F16, wq.FMT_W5E2M2, wq.FMT_W3G32,
        wq.FMT_W6E3M2_P24]
FMT_ID = {wq.FMT_W8: "w8", wq.FMT_W4G32: "w4", wq.FMT_W6E3M2: "w6", wq.FMT_W4E2M1: "fp4", wq.FMT_F16: "f16",
          wq.FMT_W5E2M2: "fp5", wq.FMT_W3G32: "w3", wq.FMT_W6E3M2_P24: "p24"}


def _weights(n, k, seed, adversarial=True):
    w, _ = inputs.small_case(seed, n, k, 1)
    if adversarial and n >= 8:
        w[0, :] = 0.0                       # zero row: scale 0
        w[1, 3] = 0.7                       # one outlier
        w[2, :] = np.abs(w[2, :])           # one-signed rows / groups
        w[3, :] = -np.abs(w[3, :])
        w[4, :32] = 1e-9                    # subnormal scale
        w[5, :] *= 1e-4                     # subnormal dequantized values
        w[6, 1] = -0.0
    return w


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_ID[f])
@pytest.mark.parametrize("n,k", [(1, 32), (15, 64), (17, 96), (64, 4096), (1000, 2080)])
def test_dequant_bit_exact(fmt, n, k):
    torch_cuda()
    w = _weights(n, k, n + k)
    dw = DeviceWeights(fmt, w)
    got = dw.dequant()
    if fmt == wq.FMT_F16:
        want = w.astype(np.float16).view(np.uint16)
    else:
        want, _, _, _ = oracle_rows(fmt, w)
    assert np.array_equal(got, want), "%d of %d differ" % (int((got != want).sum()), got.size)


@pytest.mark.parametrize("fmt,ncodes", [(wq.FMT_W6E3M2, 64), (wq.FMT_W4E2M1, 16), (wq.FMT_W5E2M2, 32),
                                        (wq.FMT_W6E3M2_P24, 64)], ids=["w6", "fp4", "fp5", "p24"])
def test_dequant_all_codes(fmt, ncodes):
    # every code in every position of a unit (codes run 0, 1, ..., shifted by one per row), at
    # scale 1, at a non-power-of-two scale and at a subnormal scale
    torch = torch_cuda()
    rows = ncodes
    codes = ((np.arange(64)[None, :] + np.arange(rows)[:, None]) % ncodes).astype(np.uint8)
    packed = oracle.pack_vectorized(fmt, codes)
    for s in (0x3C00, 0x2E66, 0x0003):
        sc = np.full(rows, s, dtype=np.uint16)
        out = torch.empty((rows, 64), dtype=torch.int16, device="cuda:0")
        wq.wq_dequant(fmt, dev(packed), dev(sc), None, out, rows, 64)
        torch.cuda.synchronize()
        want = oracle.dequant_fp16(fmt, codes, sc)
        assert np.array_equal(host_bits(out), want), hex(s)


@pytest.mark.parametrize("fmt,ncodes", [(wq.FMT_W4G32, 16), (wq.FMT_W3G32, 8)], ids=["w4", "w3"])
def test_dequant_all_codes_and_zero_points(fmt, ncodes):
    # every code in every position of a unit with every zero point, at scale 1, at a
    # non-power-of-two scale and at a subnormal scale (group g of row r: zero point (r + g) mod ncodes)
    torch = torch_cuda()
    rows, k = ncodes, 64 * ncodes
    codes = ((np.arange(k)[None, :] + np.arange(rows)[:, None]) % ncodes).astype(np.uint8)
    packed = oracle.pack_vectorized(fmt, codes)
    g = k // 32
    zeros = ((np.arange(g)[None, :] + np.arange(rows)[:, None]) % ncodes).astype(np.float16).view(np.uint16)
    for s in (0x3C00, 0x2E66, 0x0003):
        sc = np.full((rows, g), s, dtype=np.uint16)
        out = torch.empty((rows, k), dtype=torch.int16, device="cuda:0")
        wq.wq_dequant(fmt, dev(packed), dev(sc), dev(zeros), out, rows, k)
        torch.cuda.synchronize()
        want = oracle.dequant_fp16(fmt, codes, sc, zeros)
        assert np.array_equal(host_bits(out), want), hex(s)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_ID[f])
@pytest.mark.parametrize("m", list(range(1, 17)))
def test_linear_every_m(fmt, m):
    # 37 rows (ragged against 4-row and 16-row blocks); K = 4256 = 133 units: 3 chunks of
    # 64 units, the last ragged, and 34 K tiles of 4 units, the last ragged
    n, k = 37, 4256
    w = _weights(n, k, 7)
    _, x = inputs.small_case(1000 + m, 1, k, m)
    dw = DeviceWeights(fmt, w)
    wd = w.astype(np.float16).view(np.uint16) if fmt == wq.FMT_F16 else oracle_rows(fmt, w)[0]
    y = dw.linear(x)
    check_linear(y, x, wd, "fmt %d m %d" % (fmt, m))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_ID[f])
@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (1, 32, 16), (3, 64, 2), (16, 128, 5), (33, 2048, 1), (33, 2048, 9),
                                   (130, 8192, 1), (130, 8192, 16), (5, 96, 37), (64, 1024, 20), (4100, 256, 4),
                                   (16500, 128, 5),
                                   # K a multiple of 256 (W4 through LDS): a ragged last 32-unit stage
                                   # (2304 = 72 units), ragged 16-row blocks, two blocks per wave from
                                   # 8192 rows, a single stage (K = 256)
                                   (37, 2304, 5), (37, 2304, 16), (8200, 2304, 8), (40, 11008, 13), (48, 256, 6),
                                   # 17..64 rows of x in one launch (2 or 4 tiles of 16), and slabs beyond
                                   (130, 8192, 64), (37, 2304, 33), (8200, 256, 50), (40, 4352, 17), (33, 512, 130),
                                   # the plane layouts' last 64-unit chunk holding a single unit (65 units)
                                   (37, 2080, 8), (37, 2080, 20)])
def test_linear_shapes(fmt, n, k, m):
    w = _weights(n, k, 3 * n + k)
    _, x = inputs.small_case(2000 + n + m, 1, k, m)
    dw = DeviceWeights(fmt, w)
    wd = w.astype(np.float16).view(np.uint16) if fmt == wq.FMT_F16 else oracle_rows(fmt, w)[0]
    check_linear(dw.linear(x), x, wd, "fmt %d n %d k %d m %d" % (fmt, n, k, m))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_ID[f])
@pytest.mark.parametrize("m", [1, 3, 16])
def test_linear_one_hot_is_bit_exact(fmt, m):
    # x = e_k in every row: y[:, n] must equal the dequantized weight w^[n, k] exactly
    n, k = 40, 2080
    w = _weights(n, k, 11)
    dw = DeviceWeights(fmt, w)
    wd = w.astype(np.float16).view(np.uint16) if fmt == wq.FMT_F16 else oracle_rows(fmt, w)[0]
    for kk in (0, 31, 32, 1000, k - 1):
        x = np.zeros((m, k), dtype=np.float16)
        x[:, kk] = 1.0
        y = dw.linear(x.view(np.uint16))
        want = np.tile(wd[:, kk], (m, 1))
        same = (y == want) | ((y & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)   # +-0 both mean zero in a sum
        assert same.all(), (kk, np.argwhere(~same)[:3].tolist())


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_ID[f])
def test_linear_zero_x_and_repeatability(fmt):
    n, k = 70, 4096
    w = _weights(n, k, 13)
    dw = DeviceWeights(fmt, w)
    for m in (1, 16):
        y0 = dw.linear(np.zeros((m, k), dtype=np.uint16))
        assert np.all((y0 & 0x7FFF) == 0)
        _, x = inputs.small_case(77, 1, k, m)
        ys = [dw.linear(x) for _ in range(3)]
        assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_linear_rows_of_a_batch_match_single_rows():
    n, k = 48, 4096
    w = _weights(n, k, 21)
    for fmt in (wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1):
        dw = DeviceWeights(fmt, w)
        _, x = inputs.small_case(5, 1, k, 16)
        wd = oracle_rows(fmt, w)[0]
        yb = dw.linear(x)
        for i in (0, 7, 15):
            yi = dw.linear(x[i:i + 1])
            check_linear(yi, x[i:i + 1], wd)
            check_linear(yb[i:i + 1], x[i:i + 1], wd)


@pytest.mark.parametrize("n,k,m", [(8192, 8192, 4), (8192, 8192, 3), (12000, 4096, 4), (2048, 4096, 4)])
def test_w4_m4_kernel_choice_sampled(n, k, m):
    # W4 at M = 4 runs on the matrix cores from N*K = 2^24 on, on the GEMV below; both agree
    # with the oracle on sampled rows
    w, x = inputs.weights_and_x(inputs.rng_for(90, n + m), n, k, m)
    dw = DeviceWeights(wq.FMT_W4G32, w)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(n).choice(n, 62, replace=False)]))
    wd = oracle_rows(wq.FMT_W4G32, w[rows])[0]
    y = dw.linear(x)
    check_linear(y[:, rows], x, wd, "%s n %d k %d m %d" % (wq.wq_linear_kernel_name(wq.FMT_W4G32, m, n, k), n, k, m))


# ------------------------------------------------------------------ full-size workloads (sampled rows)
FULL = [
    ("w8_single_1024x1024", wq.FMT_W8),
    ("llama7b_w4g32_linears", wq.FMT_W4G32),
    ("llama70b_w6e3m2_linears", wq.FMT_W6E3M2),
    ("llama70b_w6e3m2_tp8_shard", wq.FMT_W6E3M2),
    ("llama7b_w4e2m1_linears", wq.FMT_W4E2M1),
    ("llama7b_w5e2m2_linears", wq.FMT_W5E2M2),
    ("llama7b_w8_linears", wq.FMT_W8),
    ("llama7b_w6e3m2_linears", wq.FMT_W6E3M2),
    ("llama7b_w3g32_linears", wq.FMT_W3G32),
    ("llama70b_w6e3m2_p24_linears", wq.FMT_W6E3M2_P24),
    ("llama7b_w6e3m2_p24_linears", wq.FMT_W6E3M2_P24),
]


@pytest.mark.parametrize("name,fmt", FULL, ids=[f[0] for f in FULL])
def test_workload_full_size_sampled(name, fmt):
    _, shapes, ms = inputs.WORKLOADS[name]
    stream = inputs.WORKLOAD_STREAM[name]
    mmax = max(ms)
    for li, (n, k) in enumerate(shapes):
        w, x = inputs.weights_and_x(inputs.rng_for(stream, li), n, k, mmax)
        dw = DeviceWeights(fmt, w)
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(li).choice(n, 62, replace=False)]))
        wd, codes, s, z = oracle_rows(fmt, w[rows])
        # the library's packing of these rows equals the oracle's codes
        lib_codes, _, _ = wq.wq_unpack(fmt, dw.packed_host, dw.scales_host, dw.zeros_host, n, k)
        assert np.array_equal(lib_codes[rows], codes)
        for m in ms:
            y = dw.linear(x[:m])
            check_linear(y[:, rows], x[:m], wd, "%s linear %d (%dx%d) m %d" % (name, li, n, k, m))
        del dw
        torch_cuda().cuda.empty_cache()


# ------------------------------------------------------------------ grouped launches
GROUP_SETS = {
    "mixed_k": [(40, 2080), (300, 4096), (64, 6144), (17, 96)],
    # every K a multiple of 256 (W4 through LDS), 8200 rows (two 16-row blocks per wave)
    "k256": [(40, 2304), (300, 4096), (8200, 256), (17, 512)],
}


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_ID[f])
@pytest.mark.parametrize("m", [1, 3, 4, 7, 16, 20, 40, 64, 70])
@pytest.mark.parametrize("set_name", sorted(GROUP_SETS))
def test_grouped_matches_separate_calls(fmt, m, set_name):
    torch = torch_cuda()
    shapes = GROUP_SETS[set_name]
    dws, xs = [], []
    for i, (n, k) in enumerate(shapes):
        w = _weights(n, k, 50 + i)
        dws.append(DeviceWeights(fmt, w))
        xs.append(inputs.small_case(60 + i, 1, k, m)[1])
    sep = [dw.linear(x) for dw, x in zip(dws, xs)]
    ys = [torch.zeros((m, dw.n), dtype=torch.int16, device="cuda:0") for dw in dws]
    xd = [dev(x) for x in xs]
    items = [(xd[i], dw.packed, dw.scales, dw.zeros, ys[i], dw.n, dw.k) for i, dw in enumerate(dws)]
    wq.wq_linear_grouped(items, m, fmt)
    torch.cuda.synchronize()
    grouped = wq.wq_linear_grouped_kernel_name(fmt, m, shapes)
    for i, dw in enumerate(dws):
        got = host_bits(ys[i])
        wd = dw.packed_host.view(np.uint16).reshape(dw.n, dw.k) if fmt == wq.FMT_F16 else oracle_rows(fmt, _weights(dw.n, dw.k, 50 + i))[0]
        check_linear(got, xs[i], wd, "grouped item %d" % i)
        # an item whose own plan picks the launch's kernel family and rows per wave runs the
        # same kernel body with the same K split as its separate call (or is a separate call):
        # identical bits
        own = wq.wq_linear_kernel_name(fmt, m, dw.n, dw.k)
        separate = "_grouped_kernel" not in grouped
        same_body = own.split("_kernel<")[0] == grouped.split("_grouped_kernel<")[0] and \
            own.split("<")[1] == grouped.split("<")[1]
        if separate or same_body:
            assert np.array_equal(got, sep[i]), "item %d differs from its separate call (%s, %s)" % (i, own, grouped)


def test_grouped_llama7b_w4_linears_bit_identical_to_separate_calls():
    torch = torch_cuda()
    _, shapes, _ = inputs.WORKLOADS["llama7b_w4g32_linears"]
    dws, xs, ys = [], [], []
    for li, (n, k) in enumerate(shapes):
        w, x = inputs.weights_and_x(inputs.rng_for(inputs.WORKLOAD_STREAM["llama7b_w4g32_linears"], li), n, k, 1)
        dws.append(DeviceWeights(wq.FMT_W4G32, w))
        xs.append(x)
        ys.append(torch.zeros((1, n), dtype=torch.int16, device="cuda:0"))
    items = [(dev(x), dw.packed, dw.scales, dw.zeros, y, dw.n, dw.k) for x, dw, y in zip(xs, dws, ys)]
    wq.wq_linear_grouped(items, 1, wq.FMT_W4G32)
    torch.cuda.synchronize()
    for x, dw, y in zip(xs, dws, ys):
        assert np.array_equal(host_bits(y), dw.linear(x))


def test_grouped_argument_errors():
    torch_cuda()
    L = wq.lib()
    assert L.wq_linear_grouped(None, 1, 1, 1, None) == -1
    arr = (wq.LinearItem * 17)()
    assert L.wq_linear_grouped(arr, 17, 1, 1, None) == -1
    assert L.wq_linear_grouped(arr, 0, 1, 1, None) == 0
    assert L.wq_linear_grouped(arr, 1, 1, 9, None) == -3


def test_library_loaded_before_torch_in_a_fresh_process():
    # a process whose first use of the binding is a host packer (which loads libwq.so) and
    # which imports torch only afterwards must still run its launches on torch's device memory
    import os
    import subprocess
    import sys
    code = (
        "import numpy as np\n"
        "from weight_only_quantized_dequant_amd import wq, inputs\n"
        "w, x = inputs.small_case(3, 64, 1024, 1)\n"
        "p, s = wq.wq_pack_int8(w)\n"
        "import torch\n"
        "d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16 else a).to('cuda:0')\n"
        "y = torch.empty((1, 64), dtype=torch.int16, device='cuda:0')\n"
        "wq.wq_linear(d(x), d(p), d(s), None, y, 1, 64, 1024, wq.FMT_W8, None)\n"
        "torch.cuda.synchronize()\n"
        "print('ok', int((y != 0).sum()))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split()[0] == "ok" and int(r.stdout.split()[1]) > 0, r.stdout


@pytest.mark.parametrize("n,k", [(37, 4256), (8200, 2304), (1024, 8192)])
@pytest.mark.parametrize("m", [1, 3, 4, 8, 16, 33, 70])
def test_p24_layout_gives_the_w6_outputs_bit_for_bit(n, k, m):
    # the same weights in the two FP6 layouts: the 2+4 split decodes e3m2(code) * 2^-12 and folds
    # the 2^12 into the row scale, so every fp32 sum is the W6 one scaled by a power of two and
    # the rounded outputs agree bit for bit (each kernel family against itself)
    w = _weights(n, k, 5 * n + k)
    _, x = inputs.small_case(3000 + n + m, 1, k, m)
    a, b = DeviceWeights(wq.FMT_W6E3M2, w), DeviceWeights(wq.FMT_W6E3M2_P24, w)
    assert np.array_equal(wq.wq_unpack(wq.FMT_W6E3M2, a.packed_host, a.scales_host, None, n, k)[0],
                          wq.wq_unpack(wq.FMT_W6E3M2_P24, b.packed_host, b.scales_host, None, n, k)[0])
    ya, yb = a.linear(x), b.linear(x)
    assert np.array_equal(ya, yb), "%d of %d differ (%s)" % (int((ya != yb).sum()), ya.size,
                                                            wq.wq_linear_kernel_name(wq.FMT_W6E3M2_P24, m, n, k))


# ------------------------------------------------------------------ gate/up with silu in one launch
SILU_CASES = [(1, 64, 256), (3, 64, 256), (4, 5504, 4096), (1, 5504, 4096), (2, 700, 4256), (5, 300, 2304),
              (8, 5504, 4096), (16, 4100, 2304), (33, 200, 4096), (13, 64, 4128), (70, 300, 512)]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_ID[f])
@pytest.mark.parametrize("m,f,k", SILU_CASES)
def test_linear_silu_equals_linear_then_silu_mul(fmt, m, f, k):
    # one [2F, K] matrix of interleaved gate/up rows: wq_linear_silu must give exactly what
    # wq_linear on that matrix followed by wq_silu_mul on its even and odd columns gives, wherever
    # wq_linear takes a decode kernel; and silu(gate) * up of the oracle's linear within the bound
    torch = torch_cuda()
    from oracle import decode as D
    wg, wu = _weights(f, k, 11 * f + k), _weights(f, k, 13 * f + k + 1)
    w = np.empty((2 * f, k), dtype=np.float32)
    w[0::2], w[1::2] = wg, wu
    _, x = inputs.small_case(4000 + m + f, 1, k, m)
    dw = DeviceWeights(fmt, w)
    act = torch.empty((m, f), dtype=torch.int16, device="cuda:0")
    wq.wq_linear_silu(dev(x), dw.packed, dw.scales, dw.zeros, act, m, f, k, fmt)
    torch.cuda.synchronize()
    got = host_bits(act)
    name = wq.wq_linear_kernel_name(fmt, m, 2 * f, k)
    y = dw.linear(x)
    if not name.startswith("pf_kernel"):
        n8 = (m * f + 7) // 8 * 8   # wq_silu_mul takes a multiple of 8 values: pad with zeros
        pad = lambda a: np.concatenate([np.ascontiguousarray(a).reshape(-1), np.zeros(n8 - m * f, dtype=np.uint16)])
        g, u = dev(pad(y[:, 0::2])), dev(pad(y[:, 1::2]))
        ref = torch.empty(n8, dtype=torch.int16, device="cuda:0")
        wq.wq_silu_mul(g, u, ref, n8)
        torch.cuda.synchronize()
        want = host_bits(ref)[:m * f].reshape(m, f)
        assert np.array_equal(got, want), "%d of %d differ (%s)" % (int((got != want).sum()), got.size, name)
    # against the oracle: silu(g) * u of the oracle's fp16-rounded linear outputs; the device's g and u
    # are each within the linear's bound of the oracle's, and silu * u moves that error by at most
    # |d(silu(g) u)/dg| <= 1.1 |u| and |silu(g)| in u
    wd = w.astype(np.float16).view(np.uint16) if fmt == wq.FMT_F16 else oracle_rows(fmt, w)[0]
    yref = oracle.linear_ref(x, wd)
    bound = oracle.error_bound(x, wd, yref)
    gv, uv = oracle.fp16_from_bits(oracle.fp16_bits(yref[:, 0::2])), oracle.fp16_from_bits(oracle.fp16_bits(yref[:, 1::2]))
    want = oracle.fp16_from_bits(oracle.fp16_bits(D.silu_mul(gv, uv)))
    silu = np.abs(gv / (1 + np.exp(-gv)))
    tol = (1.1 * np.abs(uv) * (bound[:, 0::2] + 2.0 ** -11 * np.abs(gv)) + (silu + 1e-3) * (bound[:, 1::2] + 2.0 ** -11 * np.abs(uv))
           + 2.0 ** -10 * np.abs(want) + 2.0 ** -24)
    err = np.abs(oracle.fp16_from_bits(got) - want)
    assert np.all(err <= tol), float((err / tol).max())


def test_linear_silu_graph_replays_match_eager():
    torch = torch_cuda()
    m, f, k = 1, 5504, 4096
    w = _weights(2 * f, k, 99)
    _, x = inputs.small_case(98, 1, k, m)
    dw = DeviceWeights(wq.FMT_W4G32, w)
    xd = dev(x)
    eager = torch.empty((m, f), dtype=torch.int16, device="cuda:0")
    wq.wq_linear_silu(xd, dw.packed, dw.scales, dw.zeros, eager, m, f, k, wq.FMT_W4G32)
    torch.cuda.synchronize()
    out = torch.zeros((m, f), dtype=torch.int16, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            wq.wq_linear_silu(xd, dw.packed, dw.scales, dw.zeros, out, m, f, k, wq.FMT_W4G32)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), host_bits(eager))


# ------------------------------------------------------------------ the largest K the library takes
@pytest.mark.parametrize("fmt", [wq.FMT_W4G32, wq.FMT_W8, wq.FMT_W6E3M2], ids=["w4", "w8", "w6"])
def test_largest_k(fmt):
    # K = 2^26 (the limit), N = 3: past K = 2^25 the decode kernels take 16-row slabs of x, so M = 17
    # runs as two launches; M = 1 takes the GEMV.
    #  * one-hot rows of x at positions spread over K (around 2^25 and at the last index): y must be
    #    the dequantized weight at that position bit for bit, which any addressing error would break;
    #  * random x: the oracle's closed-form bound, with the reference summed over K chunks in float64
    #    (the oracle's plain product, chunk by chunk, so that its memory stays bounded). The fixed
    #    rtol = atol = 1e-2 of the other tests is not applied: it suits K up to ~1e5, and a float32 sum
    #    of 2^26 terms carries absolute errors of order 0.1 on outputs of order 100.
    torch = torch_cuda()
    n, k = 3, 1 << 26
    rng = inputs.rng_for(95, fmt)
    w = (0.02 * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    dw = DeviceWeights(fmt, w)
    wd, codes, _, _ = oracle_rows(fmt, w)
    lib_codes, _, _ = wq.wq_unpack(fmt, dw.packed_host, dw.scales_host, dw.zeros_host, n, k)
    assert np.array_equal(lib_codes, codes)
    assert np.array_equal(dw.dequant(), wd)
    del lib_codes, codes, w
    pos = [0, 31, 32, 1000, (1 << 25) - 1, 1 << 25, (1 << 25) + 1, (1 << 25) + 31, (1 << 25) + 32, 3 << 24,
           k - 1025, k - 64, k - 33, k - 32, k - 31, k - 2, k - 1]
    onehot = np.zeros((len(pos), k), dtype=np.uint16)
    for i, kk in enumerate(pos):
        onehot[i, kk] = 0x3C00                      # fp16 1.0
    for rows in (onehot[:1], onehot):              # the GEMV, and two 16-row slabs
        y = dw.linear(rows)
        want = wd[:, [pos[i] for i in range(rows.shape[0])]].T
        same = (y == want) | (((y & 0x7FFF) == 0) & ((want & 0x7FFF) == 0))
        assert same.all(), (rows.shape[0], np.argwhere(~same)[:3].tolist())
    del onehot
    for m in (1, 17):
        x = rng.standard_normal((m, k), dtype=np.float32).astype(np.float16).view(np.uint16)
        y = dw.linear(x)
        yref = np.zeros((m, n))
        s_abs = np.zeros((m, n))
        a_abs = np.zeros((m, 1))
        step = 1 << 22
        for c0 in range(0, k, step):
            xc, wc = x[:, c0:c0 + step], wd[:, c0:c0 + step]
            yref += oracle.linear_ref(xc, wc)
            xa, wa = np.abs(oracle.fp16_from_bits(xc)), np.abs(oracle.fp16_from_bits(wc))
            s_abs += xa @ wa.T
            a_abs += xa.sum(axis=1, keepdims=True)
        u = 2.0 ** -11
        bound = u * np.abs(yref) + (u + k * 2.0 ** -23) * s_abs + 2.0 ** -25 * a_abs + 2.0 ** -24
        err = np.abs(oracle.fp16_from_bits(y) - yref)
        assert np.all(err <= bound), (m, wq.wq_linear_kernel_name(fmt, m, n, k), float((err / bound).max()))
    del dw
    torch.cuda.empty_cache()
