"""GPU parity of the decode-sweep configurations, at full size, launched as bench.py --sweep launches them.

One layer of a random-init Llama-2-7B (formats fp16, W8, W4, W6, FP4, FP5 at M = 1) and of a
random-init Llama-70B (W6 at M = 1, 2, 4, 8, 16): q/k/v in one grouped call, o, gate/up in one
grouped call, down, from the seeded draws the sweep uses. Sampled output rows of every linear are
checked against the oracle's own quantization of those rows (closed-form bound and rtol = atol =
1e-2), and the library's codes for those rows against the oracle's.
"""

import numpy as np
import pytest

import oracle
from weight_only_quantized_dequant_amd import inputs, wq
from tests.gpu_util import DeviceWeights, check_linear, dev, host_bits, oracle_rows, torch_cuda

pytestmark = pytest.mark.gpu

STEP_LAUNCHES = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def run_layer(model, fmt, ms):
    torch = torch_cuda()
    shapes, _, _ = inputs.SWEEP_MODELS[model]
    draws = inputs.sweep_draws(model, max(ms))
    xk = inputs.sweep_x(draws)
    weights = {nk: DeviceWeights(fmt, w) for nk, (w, _) in draws.items()}
    for (n, k), dw in weights.items():
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng([8, n, k]).choice(n, 62, replace=False)]))
        wd, codes, _, _ = oracle_rows(fmt, draws[(n, k)][0][rows])
        if fmt != wq.FMT_F16:
            lib_codes, _, _ = wq.wq_unpack(fmt, dw.packed_host, dw.scales_host, dw.zeros_host, n, k)
            assert np.array_equal(lib_codes[rows], codes), (n, k)
        dw.rows, dw.wd = rows, wd
    for m in ms:
        xd = {k: dev(x[:m]) for k, x in xk.items()}
        ys = {nm: torch.full((m, n), 0x7E00, dtype=torch.int16, device="cuda:0") for nm, n, _ in shapes}
        shape_of = {nm: (n, k) for nm, n, k in shapes}
        for names in STEP_LAUNCHES:
            items = []
            for nm in names:
                n, k = shape_of[nm]
                dw = weights[(n, k)]
                items.append((xd[k], dw.packed, dw.scales, dw.zeros, ys[nm], n, k))
            print("%s fmt %d m %d launch %s: %s" % (model, fmt, m, "/".join(names),
                  wq.wq_linear_grouped_kernel_name(fmt, m, [(it[5], it[6]) for it in items])), flush=True)
            wq.wq_linear_grouped(items, m, fmt)
        torch.cuda.synchronize()
        for nm, n, k in shapes:
            dw = weights[(n, k)]
            y = host_bits(ys[nm])
            check_linear(y[:, dw.rows], xk[k][:m], dw.wd, "%s fmt %d m %d %s (%dx%d)" % (model, fmt, m, nm, n, k))
    del weights
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [wq.FMT_F16, wq.FMT_W8, wq.FMT_W4G32, wq.FMT_W6E3M2, wq.FMT_W4E2M1, wq.FMT_W5E2M2],
                         ids=["f16", "w8", "w4", "w6", "fp4", "fp5"])
def test_llama2_7b_decode_layer_full_size_sampled(fmt):
    run_layer("llama2_7b", fmt, [1])


def test_llama70b_w6_decode_layer_full_size_sampled():
    run_layer("llama70b_w6", wq.FMT_W6E3M2, [1, 2, 4, 8, 16])
