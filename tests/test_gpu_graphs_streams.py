"""wq_linear and wq_linear_grouped on a non-default stream and under HIP graph capture.

Every kernel family (VALU GEMV, LDS-staged and fragment-load matrix-core kernels, the tiled
prefill kernel, grouped launches) is launched on a side stream inside a captured graph; the
graph is replayed several times with the program's own eager work and synchronizations in
between, and every replay must give the eager result bit for bit (the kernels use no memsets
or other capture-sensitive calls, and no atomics, so results are deterministic).
"""

import numpy as np
import pytest

from weight_only_quantized_dequant_amd import inputs, wq
from tests.gpu_util import DeviceWeights, dev, host_bits, torch_cuda

pytestmark = pytest.mark.gpu

CASES = [  # (format code, N, K, M): one of each kernel family
    (wq.FMT_W4G32, 4100, 4096, 1),        # GEMV
    (wq.FMT_W6E3M2, 2048, 4096, 3),       # GEMV
    (wq.FMT_W4G32, 2080, 4096, 9),        # LDS-staged matrix cores
    (wq.FMT_W8, 1000, 2048, 16),          # fragment-load matrix cores
    (wq.FMT_W4E2M1, 300, 2080, 40),       # LDS-staged, several 16-row tiles
    (wq.FMT_W6E3M2, 1000, 2048, 300),     # tiled prefill
    (wq.FMT_W4G32 | wq.ACT_BF16, 700, 2048, 5),
]


def _case(fmt, n, k, m, seed):
    w, x = inputs.small_case(seed, n, k, m)
    if fmt & wq.ACT_BF16:
        torch = torch_cuda()
        x = torch.from_numpy(x.view(np.float16).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    return DeviceWeights(fmt & 0xFF, w, fmt & wq.ACT_BF16), x


@pytest.mark.parametrize("fmt,n,k,m", CASES, ids=["w4-gemv", "w6-gemv", "w4-lm", "w8-mfma", "fp4-lm40", "w6-prefill",
                                                   "w4bf16-lm"])
def test_linear_side_stream_and_graph_replays(fmt, n, k, m):
    torch = torch_cuda()
    dw, x = _case(fmt, n, k, m, 900 + m)
    eager = dw.linear(x)
    xd = dev(x)
    y = torch.empty((m, n), dtype=torch.int16, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # a plain launch on the side stream first
        wq.wq_linear(xd, dw.packed, dw.scales, dw.zeros, y, m, n, k, fmt, side)
    side.synchronize()
    assert np.array_equal(host_bits(y), eager)
    g = torch.cuda.CUDAGraph()
    y.zero_()
    with torch.cuda.graph(g, stream=side):
        wq.wq_linear(xd, dw.packed, dw.scales, dw.zeros, y, m, n, k, fmt, side)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(rep + 1)                             # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), eager), "replay %d" % rep


@pytest.mark.parametrize("fmt,m", [(wq.FMT_W4G32, 1), (wq.FMT_W6E3M2, 8), (wq.FMT_W4E2M1, 260)],
                         ids=["gemv", "lm", "prefill"])
def test_grouped_graph_replays(fmt, m):
    torch = torch_cuda()
    shapes = [(1040, 4096), (300, 2048), (2100, 4096)]
    dws, xs = [], []
    for i, (n, k) in enumerate(shapes):
        dw, x = _case(fmt, n, k, m, 950 + i)
        dws.append(dw)
        xs.append(x)
    xd = [dev(x) for x in xs]
    ys = [torch.zeros((m, dw.n), dtype=torch.int16, device="cuda:0") for dw in dws]
    items = [(xd[i], dw.packed, dw.scales, dw.zeros, ys[i], dw.n, dw.k) for i, dw in enumerate(dws)]
    wq.wq_linear_grouped(items, m, fmt)   # the eager grouped result on the current stream
    torch.cuda.synchronize()
    eager = [host_bits(y) for y in ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        wq.wq_linear_grouped(items, m, fmt, side)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.fill_(7 * rep + 1)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            assert np.array_equal(host_bits(y), eager[i]), "replay %d item %d" % (rep, i)
