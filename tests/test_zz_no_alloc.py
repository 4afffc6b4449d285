"""The no-allocation attention entry point (wq_rope_attention_noalloc) against wq_rope_attention.

Two calls in a row through the C ABI, the second with smaller sizes, each compared bit for bit
(output and both caches) with wq_rope_attention given its own freshly allocated workspace on the
same inputs; and sizes beyond the library's scratch buffer rejected before any launch.
"""

import ctypes

import numpy as np
import pytest

from weight_only_quantized_dequant_amd import wq
from tests.gpu_util import dev, host_bits, torch_cuda

pytestmark = pytest.mark.gpu


def _inputs(m, H, Hkv, hd, S, seed):
    rng = np.random.default_rng([seed, m, H, Hkv, hd, S])
    f = lambda *shape: rng.standard_normal(shape).astype(np.float16).view(np.uint16)
    return f(m, H * hd), f(m, Hkv * hd), f(m, Hkv * hd), f(m, S, Hkv * hd), f(m, S, Hkv * hd)


def _call(noalloc, m, H, Hkv, hd, S, p, seed):
    torch = torch_cuda()
    q, k, v, ck, cv = _inputs(m, H, Hkv, hd, S, seed)
    cos, sin = wq.wq_rope_table(10000.0, hd, S)
    ckd, cvd = dev(ck.reshape(-1)), dev(cv.reshape(-1))
    out = torch.empty(m * H * hd, dtype=torch.int16, device="cuda:0")
    pos = torch.tensor([p], dtype=torch.int32, device="cuda:0")
    args = (dev(q), dev(k), dev(v), ckd, cvd, torch.from_numpy(cos.reshape(-1)).to("cuda:0"),
            torch.from_numpy(sin.reshape(-1)).to("cuda:0"), pos, out, m, H, Hkv, hd, S)
    if noalloc:
        wq.wq_rope_attention_noalloc(*args)
    else:
        ws = wq.wq_attention_workspace_bytes(m, H, hd, S)
        wq.wq_rope_attention(*args, torch.zeros(max(ws, 16), dtype=torch.uint8, device="cuda:0") if ws else None)
    torch.cuda.synchronize()
    return host_bits(out), host_bits(ckd), host_bits(cvd)


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    cases = [(2, 16, 4, 128, 8192, 6000, 1),   # 94 chunks: partial results through the scratch buffer
             (1, 8, 2, 64, 4608, 4200, 2)]     # smaller, right after it on the same buffer
    got = [_call(True, *c) for c in cases]
    for c, g in zip(cases, got):
        want = _call(False, *c)
        for a, b in zip(g, want):
            assert np.array_equal(a, b), c


def test_noalloc_short_cache_needs_no_scratch():
    c = (3, 4, 4, 128, 64, 40, 3)
    assert wq.wq_attention_workspace_bytes(*c[0:2], c[3], c[4]) == 0
    for a, b in zip(_call(True, *c), _call(False, *c)):
        assert np.array_equal(a, b)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    torch = torch_cuda()
    m, H, hd, S = 64, 64, 128, 8192
    assert wq.wq_attention_workspace_bytes(m, H, hd, S) > wq.NOALLOC_SCRATCH_BYTES
    a = torch.zeros(1 << 10, dtype=torch.int16, device="cuda:0")
    pa = ctypes.c_void_p(a.data_ptr())
    st = wq.lib().wq_rope_attention_noalloc(pa, pa, pa, pa, pa, pa, pa, pa, pa, m, H, H, hd, S, None)
    assert st == -8 and wq.wq_status_string(st).startswith("sizes exceed")
