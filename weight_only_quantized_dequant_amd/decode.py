"""A whole decode step of a Llama-style model through libwq's C ABI, capturable as one HIP graph.

Argument marshalling only: every step of the model runs in libwq's kernels (wq_embed,
wq_add_rmsnorm, wq_linear_grouped / wq_linear on the packed weights, wq_rope_attention,
wq_linear_silu for gate/up and silu(gate)*up in one launch, wq_argmax_next). torch provides device memory, the stream and the HIP graph that
records one step. The position and the token ids live in device memory and wq_argmax_next
advances them, so replaying the graph generates token after token.

The gpt-fast write-up (m.greenbasetech.com, part on torch.compile) is the motivation for the
captured step: the CPU cannot feed the GPU launch by launch fast enough, so the whole step is
issued as one region. The speed-up strategies page (sharktoolz.top, section 6) is the source of
the key/value cache with query heads sharing key/value heads.
"""

import numpy as np

from . import inputs, wq

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
# The linears as the device holds them: gate and up as one matrix of interleaved rows (row 2i
# gate row i, row 2i+1 up row i) for wq_linear_silu.
DEVICE_LINEARS = ("q", "k", "v", "o", "gu", "down")

# Llama-2-7B decoder shapes (random-init weights of this architecture stand in for trained ones)
LLAMA2_7B = dict(d=4096, n_heads=32, n_kv_heads=32, hd=128, ffn=11008, layers=32, vocab=32000, eps=1e-5,
                 theta=10000.0)


def linear_shapes(cfg):
    """(name, N, K) of the linears of one layer."""
    d, hd, ffn = cfg["d"], cfg["hd"], cfg["ffn"]
    return [("q", cfg["n_heads"] * hd, d), ("k", cfg["n_kv_heads"] * hd, d), ("v", cfg["n_kv_heads"] * hd, d),
            ("o", d, cfg["n_heads"] * hd), ("gate", ffn, d), ("up", ffn, d), ("down", d, ffn)]


def device_shapes(cfg):
    """{name: (N, K)} of the linears as the device holds them (DEVICE_LINEARS)."""
    s = {nm: (n, k) for nm, n, k in linear_shapes(cfg)}
    s["gu"] = (2 * cfg["ffn"], cfg["d"])
    return {nm: s[nm] for nm in DEVICE_LINEARS}


def interleave_rows(a, b):
    """[F, K] and [F, K] -> [2F, K] with row 2i = a[i], row 2i+1 = b[i]."""
    out = np.empty((2 * a.shape[0], a.shape[1]), dtype=a.dtype)
    out[0::2], out[1::2] = a, b
    return out


def pack_host(fmt, w):
    """Quantize + pack fp32 W [N,K] with libwq's host packers: (packed, scales, zeros) numpy arrays."""
    fmt &= 0xFF
    if fmt == wq.FMT_W8:
        return wq.wq_pack_int8(w) + (None,)
    if fmt == wq.FMT_W4G32:
        return wq.wq_pack_int4(w)
    if fmt == wq.FMT_W6E3M2:
        return wq.wq_pack_fp6(w) + (None,)
    if fmt == wq.FMT_W4E2M1:
        return wq.wq_pack_fp4(w) + (None,)
    if fmt == wq.FMT_W5E2M2:
        return wq.wq_pack_fp5(w) + (None,)
    if fmt == wq.FMT_W3G32:
        return wq.wq_pack_int3(w)
    if fmt == wq.FMT_W6E3M2_P24:
        return wq.wq_pack_fp6_p24(w) + (None,)
    if fmt == wq.FMT_F16:
        return np.asarray(w, dtype=np.float32).astype(np.float16).view(np.uint8).reshape(-1), None, None
    raise ValueError("format %r" % fmt)


class Decoder:
    """Device state of a model and one decode step of M sequences (all at the same position).

    layers: list over layers of dicts: each name of DEVICE_LINEARS -> host packed tuple (packed,
    scales, zeros), 'attn_norm' / 'ffn_norm' -> fp16 bits [d]. final_norm: fp16 bits [d]; lm_head: packed
    tuple [vocab, d]; embed: fp16 bits [vocab, d]. Every layer gets its own device copy of its
    arrays (layers that share host arrays still stream their own bytes, as a real model would)."""

    def __init__(self, torch, cfg, fmt, m, max_seq, layers, final_norm, lm_head, embed, device="cuda"):
        self.torch, self.cfg, self.fmt, self.m, self.S = torch, cfg, fmt, m, max_seq
        dev = lambda a: None if a is None else torch.from_numpy(
            np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(device)
        d, hd, H, Hkv, ffn, V = cfg["d"], cfg["hd"], cfg["n_heads"], cfg["n_kv_heads"], cfg["ffn"], cfg["vocab"]
        self.shapes = device_shapes(cfg)
        self.layers = []
        for L in layers:
            self.layers.append({nm: tuple(dev(a) for a in L[nm]) for nm in DEVICE_LINEARS})
            self.layers[-1]["attn_norm"] = dev(L["attn_norm"])
            self.layers[-1]["ffn_norm"] = dev(L["ffn_norm"])
        self.final_norm = dev(final_norm)
        self.lm_head = tuple(dev(a) for a in lm_head)
        self.embed = dev(embed)
        empty = lambda n, dt=torch.int16: torch.zeros(n, dtype=dt, device=device)
        self.x = empty(m * d, torch.float32)
        self.h = empty(m * d)
        self.q, self.att = empty(m * H * hd), empty(m * H * hd)
        self.k, self.v = empty(m * Hkv * hd), empty(m * Hkv * hd)
        self.o, self.down = empty(m * d), empty(m * d)
        self.act = empty(m * ffn)
        self.logits = empty(m * V)
        self.tokens = empty(m, torch.int32)
        self.pos = empty(1, torch.int32)
        self.cache_k = [empty(m * max_seq * Hkv * hd) for _ in layers]
        self.cache_v = [empty(m * max_seq * Hkv * hd) for _ in layers]
        cos, sin = wq.wq_rope_table(cfg["theta"], hd, max_seq)
        self.rope_cos, self.rope_sin = torch.from_numpy(cos.reshape(-1)).to(device), torch.from_numpy(sin.reshape(-1)).to(device)
        ws = wq.wq_attention_workspace_bytes(m, H, hd, max_seq)
        self.workspace = empty(max(ws, 16), torch.uint8) if ws else None

    def launches_per_step(self):
        """Kernel launches of one step: embedding, final norm, output layer, next token, and per layer two
        norms, q/k/v, attention (and its combine launch when the cache holds more than one chunk), o,
        gate/up with silu, down."""
        return 4 + len(self.layers) * (7 + (1 if self.workspace is not None else 0))

    def weight_bytes(self):
        """Bytes of packed weights and metadata one step reads (layers and output layer)."""
        f = self.fmt & 0xFF
        per = sum(wq.wq_packed_bytes(f, n, k) + wq.wq_scales_bytes(f, n, k) + wq.wq_zeros_bytes(f, n, k)
                  for n, k in self.shapes.values())
        V, d = self.cfg["vocab"], self.cfg["d"]
        return per * len(self.layers) + wq.wq_packed_bytes(f, V, d) + wq.wq_scales_bytes(f, V, d) + wq.wq_zeros_bytes(f, V, d)

    def _item(self, L, nm, x, y):
        p, s, z = L[nm]
        n, k = self.shapes[nm]
        return (x, p, s, z, y, n, k)

    def step(self, stream=None):
        """Issue one decode step: tokens at pos -> logits, next tokens, pos + 1."""
        c, m, f = self.cfg, self.m, self.fmt
        d, hd, H, Hkv, ffn, V = c["d"], c["hd"], c["n_heads"], c["n_kv_heads"], c["ffn"], c["vocab"]
        wq.wq_embed(self.embed, self.tokens, self.x, m, d, V, stream)
        delta = None
        for l, L in enumerate(self.layers):
            wq.wq_add_rmsnorm(self.x, delta, L["attn_norm"], c["eps"], self.h, m, d, stream)
            wq.wq_linear_grouped([self._item(L, "q", self.h, self.q), self._item(L, "k", self.h, self.k),
                                  self._item(L, "v", self.h, self.v)], m, f, stream)
            wq.wq_rope_attention(self.q, self.k, self.v, self.cache_k[l], self.cache_v[l], self.rope_cos, self.rope_sin,
                                 self.pos, self.att, m, H, Hkv, hd, self.S, self.workspace, stream)
            wq.wq_linear_grouped([self._item(L, "o", self.att, self.o)], m, f, stream)
            wq.wq_add_rmsnorm(self.x, self.o, L["ffn_norm"], c["eps"], self.h, m, d, stream)
            p, s, z = L["gu"]
            wq.wq_linear_silu(self.h, p, s, z, self.act, m, ffn, d, f, stream)
            wq.wq_linear_grouped([self._item(L, "down", self.act, self.down)], m, f, stream)
            delta = self.down
        wq.wq_add_rmsnorm(self.x, delta, self.final_norm, c["eps"], self.h, m, d, stream)
        p, s, z = self.lm_head
        wq.wq_linear(self.h, p, s, z, self.logits, m, V, d, f, stream)
        wq.wq_argmax_next(self.logits, m, V, self.tokens, self.pos, stream)

    def capture(self):
        """One step recorded as a HIP graph (on a side stream); replay() runs the next step."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.step()
        torch.cuda.current_stream().wait_stream(s)
        return g


def random_model(cfg, fmt, stream_id, distinct_layers=None):
    """Seeded random-init weights of cfg's shapes, packed by libwq. With distinct_layers = k, the first
    k layers get their own draws and the rest repeat them in turn (time depends only on shapes and
    bytes; each layer still gets its own device memory). Returns (layers, final_norm, lm_head, embed)
    as host arrays, and the fp32 draws {(layer, name): W} for an oracle."""
    nl = cfg["layers"]
    k = nl if distinct_layers is None else min(distinct_layers, nl)
    d, V = cfg["d"], cfg["vocab"]
    draws, packed = {}, []
    for l in range(k):
        rng = inputs.rng_for(stream_id, l)
        L = {}
        for nm, n, kk in linear_shapes(cfg):
            w = (0.02 * rng.standard_normal((n, kk), dtype=np.float32)).astype(np.float32)
            draws[(l, nm)] = w
            if nm not in ("gate", "up"):
                L[nm] = pack_host(fmt, w)
        L["gu"] = pack_host(fmt, interleave_rows(draws[(l, "gate")], draws[(l, "up")]))
        L["attn_norm"] = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float16).view(np.uint16)
        L["ffn_norm"] = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float16).view(np.uint16)
        draws[(l, "attn_norm")], draws[(l, "ffn_norm")] = L["attn_norm"], L["ffn_norm"]
        packed.append(L)
    layers = [packed[l % k] for l in range(nl)]
    rng = inputs.rng_for(stream_id, 1000)
    w_out = (0.02 * rng.standard_normal((V, d), dtype=np.float32)).astype(np.float32)
    draws["lm_head"] = w_out
    final_norm = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float16).view(np.uint16)
    embed = rng.standard_normal((V, d), dtype=np.float32).astype(np.float16).view(np.uint16)
    draws["final_norm"], draws["embed"] = final_norm, embed
    return (layers, final_norm, pack_host(fmt, w_out), embed), draws
