"""GPU parity of the tiled prefill kernel against the oracle (wq_linear from 193 rows of x on, and
from 65 rows on for linears with enough tiles for their chain of K steps).

The kernel stages 128 x 128 tiles of x and of the decoded weights in LDS; these cases cover
ragged tiles in M and N, K with an odd number of 32-code units (a half-empty last K step),
every weight format with fp16 and with bfloat16 activations, one-hot x (bit-exact), grouped
launches (bit-identical to separate calls), and the Llama-7B shapes at M = 512 on sampled
output rows.
"""

import numpy as np
import pytest

from weight_only_quantized_dequant_amd import inputs, wq
from tests.gpu_util import (DeviceWeights, bf16_bits_torch, check_linear, dev, host_bits, oracle_rows, torch_cuda,
                            x_as_bf16)

pytestmark = pytest.mark.gpu

BF = wq.ACT_BF16
CODES = [(wq.FMT_F16, 0), (wq.FMT_W8, 0), (wq.FMT_W4G32, 0), (wq.FMT_W6E3M2, 0), (wq.FMT_W4E2M1, 0),
         (wq.FMT_W8, BF), (wq.FMT_W4G32, BF), (wq.FMT_W6E3M2, BF), (wq.FMT_W4E2M1, BF), (wq.FMT_BF16, BF),
         (wq.FMT_W5E2M2, 0), (wq.FMT_W5E2M2, BF), (wq.FMT_W3G32, 0), (wq.FMT_W6E3M2_P24, 0)]
NAMES = {wq.FMT_F16: "f16", wq.FMT_W8: "w8", wq.FMT_W4G32: "w4", wq.FMT_W6E3M2: "w6", wq.FMT_W4E2M1: "fp4",
         wq.FMT_BF16: "bf16w", wq.FMT_W5E2M2: "fp5", wq.FMT_W3G32: "w3", wq.FMT_W6E3M2_P24: "p24"}
IDS = ["%s%s" % (NAMES[f], "_bf16" if a else "") for f, a in CODES]


def _weights(n, k, seed):
    w, _ = inputs.small_case(seed, n, k, 1)
    if n >= 8:
        w[0, :] = 0.0
        w[1, 3] = 0.7
        w[2, :] = np.abs(w[2, :])
        w[4, :32] = 1e-9
        w[5, :] *= 1e-4
    return w


def _ref(fmt, act, w):
    if fmt == wq.FMT_F16:
        return w.astype(np.float16).view(np.uint16)
    if fmt == wq.FMT_BF16:
        return bf16_bits_torch(w)
    return oracle_rows(fmt, w, act)[0]


def _x(seed, k, m, act):
    x = inputs.small_case(seed, 1, k, m)[1]
    return x_as_bf16(x) if act == BF else x


@pytest.mark.parametrize("fmt,act", CODES, ids=IDS)
@pytest.mark.parametrize("n,k,m", [(1, 32, 193), (100, 96, 256), (130, 2080, 300), (257, 4256, 600), (64, 4096, 700),
                                   (200, 256, 1030), (8200, 256, 512), (33, 11008, 512), (129, 2048, 200),
                                   (4100, 256, 100), (3000, 512, 150), (9000, 96, 65)])
def test_prefill_shapes(fmt, act, n, k, m):
    w = _weights(n, k, 7 * n + k)
    x = _x(5000 + n + m, k, m, act)
    dw = DeviceWeights(fmt, w, act)
    name = wq.wq_linear_kernel_name(fmt | act, m, n, k)
    # from 193 rows always the tiled kernel; below, the planner may keep a decode kernel (FP5
    # leaves the decode kernels only from 81 rows, and then not on every shape): parity either way
    assert name.startswith("pf_kernel") or (m < 193 and fmt == wq.FMT_W5E2M2), name
    check_linear(dw.linear(x), x, _ref(fmt, act, w), "fmt %d act %d n %d k %d m %d" % (fmt, act, n, k, m), act=act)


W8_F16 = [(f, a) for f, a in CODES if f in (wq.FMT_F16, wq.FMT_W8, wq.FMT_BF16)]


@pytest.mark.parametrize("fmt,act", W8_F16, ids=["%s%s" % (NAMES[f], "_bf16" if a else "") for f, a in W8_F16])
@pytest.mark.parametrize("n,k,m", [(16600, 256, 48), (16500, 128, 24), (12000, 1024, 57)])
def test_prefill_small_m_w8_and_16bit_weights(fmt, act, n, k, m):
    # W8 and fp16/bf16 weights below 65 rows of x: the tiled kernel where its K chain is short
    w = _weights(n, k, 3 * n + k)
    x = _x(6000 + n + m, k, m, act)
    dw = DeviceWeights(fmt, w, act)
    assert wq.wq_linear_kernel_name(fmt | act, m, n, k).startswith("pf_kernel")
    check_linear(dw.linear(x), x, _ref(fmt, act, w), "fmt %d act %d n %d k %d m %d" % (fmt, act, n, k, m), act=act)


@pytest.mark.parametrize("fmt,act", CODES, ids=IDS)
def test_prefill_one_hot_is_bit_exact(fmt, act):
    n, k, m = 150, 2080, 520
    w = _weights(n, k, 11)
    dw = DeviceWeights(fmt, w, act)
    wd = _ref(fmt, act, w)
    one = 0x3F80 if act == BF else 0x3C00
    x = np.zeros((m, k), dtype=np.uint16)
    cols = (np.arange(m) * 37) % k                  # a different column in every row of x
    x[np.arange(m), cols] = one
    y = dw.linear(x)
    want = wd[:, cols].T
    same = (y == want) | ((y & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
    assert same.all(), np.argwhere(~same)[:3].tolist()


@pytest.mark.parametrize("fmt,act", CODES, ids=IDS)
def test_prefill_repeatable_and_rows_independent(fmt, act):
    # a row of x gives the same y inside a 512-row call and inside a 700-row call
    n, k = 90, 4096
    w = _weights(n, k, 13)
    dw = DeviceWeights(fmt, w, act)
    x = _x(91, k, 700, act)
    y700 = dw.linear(x)
    assert np.array_equal(y700, dw.linear(x))
    y512 = dw.linear(x[100:612])
    assert np.array_equal(y700[100:612], y512)


@pytest.mark.parametrize("fmt,act", CODES, ids=IDS)
@pytest.mark.parametrize("m", [193, 520])
def test_prefill_grouped_matches_separate_calls(fmt, act, m):
    # one launch over the tiles of every item (mixed K, ragged N, an odd number of K units):
    # each item's y bit-identical to its own call, and within tolerance of the oracle
    torch = torch_cuda()
    shapes = [(130, 2080), (300, 4096), (64, 6144), (17, 96), (257, 4256)]
    ws = [_weights(n, k, 60 + i) for i, (n, k) in enumerate(shapes)]
    dws = [DeviceWeights(fmt, w, act) for w in ws]
    xs = [_x(70 + i, k, m, act) for i, (_, k) in enumerate(shapes)]
    sep = [dw.linear(x) for dw, x in zip(dws, xs)]
    xd = [dev(x) for x in xs]
    ys = [torch.empty((m, dw.n), dtype=torch.int16, device="cuda:0") for dw in dws]
    items = [(xd[i], dw.packed, dw.scales, dw.zeros, ys[i], dw.n, dw.k) for i, dw in enumerate(dws)]
    assert wq.wq_linear_grouped_kernel_name(fmt | act, m, shapes) == "pf_grouped_kernel<%d>" % (fmt | act)
    wq.wq_linear_grouped(items, m, fmt | act)
    torch.cuda.synchronize()
    for i, (w, x) in enumerate(zip(ws, xs)):
        got = host_bits(ys[i])
        assert np.array_equal(got, sep[i]), "item %d differs from its separate call" % i
        check_linear(got, x, _ref(fmt, act, w), "grouped item %d m %d" % (i, m), act=act)


@pytest.mark.parametrize("fmt,act", [(wq.FMT_W4G32, 0), (wq.FMT_W6E3M2, 0), (wq.FMT_W4G32, BF)],
                         ids=["w4", "w6", "w4_bf16"])
def test_prefill_llama7b_m512_sampled(fmt, act):
    _, shapes, _ = inputs.WORKLOADS["llama7b_w4g32_linears"]
    for li, (n, k) in enumerate(shapes):
        w, x16 = inputs.weights_and_x(inputs.rng_for(40, li), n, k, 512)
        x = x_as_bf16(x16) if act == BF else x16
        dw = DeviceWeights(fmt, w, act)
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(li).choice(n, 62, replace=False)]))
        wd = oracle_rows(fmt, w[rows], act)[0]
        y = dw.linear(x)
        check_linear(y[:, rows], x, wd, "linear %d (%dx%d) m 512" % (li, n, k), act=act)
        del dw
        torch_cuda().cuda.empty_cache()
