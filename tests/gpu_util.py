"""Marshalling helpers for the GPU tests: numpy host arrays <-> torch device buffers, and oracle comparisons."""

import numpy as np

import oracle
from weight_only_quantized_dequant_amd import wq


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU; torch.cuda.is_available() is False")
    return torch


def dev(a):
    """numpy array -> contiguous torch tensor on cuda:0 with the same bytes."""
    torch = torch_cuda()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a.copy()).to("cuda:0")


def host_bits(t):
    """torch fp16/int16 device tensor -> numpy uint16 bit patterns."""
    torch = torch_cuda()
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_bits_torch(a):
    """float array -> bfloat16 bit patterns, rounded by torch (float32 -> bfloat16, nearest even)."""
    import torch
    f = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def x_as_bf16(x16_bits):
    """fp16 activations from the seeded generators -> the same values rounded to bfloat16."""
    return bf16_bits_torch(np.asarray(x16_bits, dtype=np.uint16).view(np.float16).astype(np.float32))


def pack_with_library(fmt, w):
    """Quantize + pack on the host with libwq. Returns (packed, scales, zeros) numpy arrays."""
    if fmt == wq.FMT_W8:
        p, s = wq.wq_pack_int8(w)
        return p, s, None
    if fmt == wq.FMT_W4G32:
        return wq.wq_pack_int4(w)
    if fmt == wq.FMT_W6E3M2:
        p, s = wq.wq_pack_fp6(w)
        return p, s, None
    if fmt == wq.FMT_W4E2M1:
        p, s = wq.wq_pack_fp4(w)
        return p, s, None
    if fmt == wq.FMT_W5E2M2:
        p, s = wq.wq_pack_fp5(w)
        return p, s, None
    if fmt == wq.FMT_W3G32:
        return wq.wq_pack_int3(w)
    if fmt == wq.FMT_W6E3M2_P24:
        p, s = wq.wq_pack_fp6_p24(w)
        return p, s, None
    if fmt == wq.FMT_F16:
        return np.asarray(w, dtype=np.float32).astype(np.float16).view(np.uint8).reshape(-1), None, None
    if fmt == wq.FMT_BF16:
        return bf16_bits_torch(w).view(np.uint8).reshape(-1), None, None
    raise ValueError(fmt)


class DeviceWeights:
    """Packed weights of one linear, uploaded to the device. act: wq.ACT_F16 or wq.ACT_BF16."""

    def __init__(self, fmt, w, act=wq.ACT_F16):
        self.fmt = fmt
        self.code = fmt | act
        self.n, self.k = w.shape
        p, s, z = pack_with_library(fmt, w)
        self.packed_host, self.scales_host, self.zeros_host = p, s, z
        self.packed = dev(p)
        self.scales = dev(s) if s is not None else None
        self.zeros = dev(z) if z is not None else None

    def linear(self, x_bits, stream=None):
        torch = torch_cuda()
        m = x_bits.shape[0]
        x = dev(x_bits)
        y = torch.empty((m, self.n), dtype=torch.int16, device="cuda:0")
        wq.wq_linear(x, self.packed, self.scales, self.zeros, y, m, self.n, self.k, self.code, stream)
        torch.cuda.synchronize()
        return host_bits(y)

    def dequant(self):
        torch = torch_cuda()
        out = torch.empty((self.n, self.k), dtype=torch.int16, device="cuda:0")
        wq.wq_dequant(self.code, self.packed, self.scales, self.zeros, out, self.n, self.k)
        torch.cuda.synchronize()
        return host_bits(out)


def oracle_rows(fmt, w_rows, act=wq.ACT_F16):
    """Oracle quantize + dequant for some rows: (dequantized bits, codes, scales, zeros); the
    dequantized weights are fp16, or bfloat16 with act = wq.ACT_BF16."""
    _, s, z, codes = oracle.quantize_and_pack(fmt, w_rows)
    if act == wq.ACT_BF16:
        return oracle.dequant_bf16(fmt, codes, s, z), codes, s, z
    return oracle.dequant_fp16(fmt, codes, s, z), codes, s, z


def check_linear(y_bits, x_bits, wd_bits, what="", act=wq.ACT_F16, fixed_tol=True):
    """Device y against the oracle: the closed-form bound and rtol = atol = 1e-2 (fp16 bits). With
    act = wq.ACT_BF16 (bfloat16 bits) the fixed tolerance is 8e-2: the fp16 one scaled by the ratio
    of the unit roundoffs, 2^-8 / 2^-11. fixed_tol=False keeps only the bound, which scales with
    the data (the fixed atol suits inputs of order one)."""
    a = oracle.ACT_BF16 if act == wq.ACT_BF16 else oracle.ACT_F16
    yref = oracle.linear_ref(x_bits, wd_bits, act=a)
    bound = oracle.error_bound(x_bits, wd_bits, yref, act=a)
    y = oracle.bf16_from_bits(y_bits) if act == wq.ACT_BF16 else oracle.fp16_from_bits(y_bits)
    err = np.abs(y - yref)
    assert np.all(np.isfinite(y)), what
    bad = err > bound
    assert not bad.any(), "%s: %d of %d outside the bound; worst err %g (bound %g) at %s" % (
        what, int(bad.sum()), bad.size, float(err[bad].max()), float(bound[bad][np.argmax(err[bad])]),
        np.argwhere(bad)[0].tolist())
    if fixed_tol:
        tol = 8e-2 if act == wq.ACT_BF16 else 1e-2
        lim = tol + tol * np.abs(yref)
        assert np.all(err <= lim), "%s: worst err / (atol + rtol |y|) = %g" % (what, float((err / lim).max()))
    return float((err / np.maximum(bound, 1e-30)).max())
