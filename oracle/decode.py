"""Reference decode step of a Llama-style model built around the weight-only-quantized linears.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The pages name the loop around the linear layer without defining it: the gpt-fast write-up
(m.greenbasetech.com, part on torch.compile) runs a whole decode step as one captured region
so that the CPU stops feeding the GPU piece by piece, and reloads every weight once per
generated token (part on GPU quantization); the speed-up strategies page (sharktoolz.top,
section 6 "KV cache and multi-query attention") keeps the keys and values of processed tokens
in a cache and lets several query heads share one key/value head. The model around the
linears is read as the Llama decoder layer those pages discuss, with its usual definitions:

* RMSNorm: ``out_i = x_i * g_i / sqrt(mean_j(x_j^2) + eps)``.
* Rotary position embedding on consecutive pairs ``(x[2i], x[2i+1])`` of a head of size
  ``hd``: rotation by the angle ``pos * theta^(-2i/hd)``.
* Attention of one new token over the cached positions ``0..pos``: scores
  ``q.k_t / sqrt(hd)``, softmax, weighted sum of the values; query head ``h`` reads key/value
  head ``h // (H / H_kv)``.
* Feed-forward ``down(silu(gate(h)) * up(h))`` with ``silu(g) = g / (1 + e^-g)``.
* Residual stream ``x += attention_out`` and ``x += ffn_out``; final RMSNorm; output linear;
  the next token is the lowest index of the largest logit.

Precision. Everything is computed in float64. Where the device path stores a value in fp16
(the normalised activations, every linear output, the rotated keys and the values in the
cache, the attention output, silu(gate)*up, the logits) the reference rounds it to fp16 at the
same point, so that the two paths see the same kind of inputs at every step. The residual
stream stays unrounded here (the device keeps it in fp32).
"""

import numpy as np

from .formats import fp16_bits, fp16_from_bits
from .linear import dequant_fp16, linear_ref


def f16(a):
    """Round float64 values to fp16 and return them as float64 (the value the device stores)."""
    return fp16_from_bits(fp16_bits(a))


def rmsnorm(x, g, eps):
    """x [M, d] float64, g [d] (fp16 values) -> fp16 values [M, d]."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return f16(x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64))


def rope_angles(pos, hd, theta):
    """The angles of the hd/2 pairs of a head at position pos: pos * theta^(-2i/hd)."""
    i = np.arange(hd // 2, dtype=np.float64)
    return float(pos) * np.power(float(theta), -2.0 * i / hd)


def rope(x, pos, hd, theta):
    """Rotate each head (consecutive hd values) of x [M, heads*hd] at position pos, pairs (2i, 2i+1)."""
    x = np.asarray(x, dtype=np.float64)
    m, w = x.shape
    h = x.reshape(m, w // hd, hd // 2, 2)
    a = rope_angles(pos, hd, theta)
    c, s = np.cos(a), np.sin(a)
    x0, x1 = h[..., 0], h[..., 1]
    out = np.stack([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)
    return out.reshape(m, w)


def attention(q, cache_k, cache_v, pos, n_heads, n_kv_heads, hd):
    """One query token per sequence over positions 0..pos of its cache.

    q [M, n_heads*hd] (rotated), cache_k / cache_v [M, S, n_kv_heads*hd] (values as stored).
    Returns the output [M, n_heads*hd] before the fp16 rounding.
    """
    q = np.asarray(q, dtype=np.float64)
    m = q.shape[0]
    group = n_heads // n_kv_heads
    out = np.zeros((m, n_heads * hd))
    for b in range(m):
        for h in range(n_heads):
            kv = h // group
            qh = q[b, h * hd:(h + 1) * hd]
            k = np.asarray(cache_k[b, :pos + 1, kv * hd:(kv + 1) * hd], dtype=np.float64)
            v = np.asarray(cache_v[b, :pos + 1, kv * hd:(kv + 1) * hd], dtype=np.float64)
            s = k @ qh / np.sqrt(hd)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, h * hd:(h + 1) * hd] = p @ v
    return out


def silu_mul(g, u):
    """fp16 values g, u -> fp16 values of g / (1 + e^-g) * u."""
    g = np.asarray(g, dtype=np.float64)
    return f16(g / (1.0 + np.exp(-g)) * np.asarray(u, dtype=np.float64))


def argmax_lowest(logits):
    """Per row, the lowest index of the largest value."""
    return np.argmax(np.asarray(logits, dtype=np.float64), axis=1).astype(np.int32)


class Model:
    """A Llama-style model for the reference: per layer the quantized linears (as dequantized fp16
    bit arrays, from the oracle's own quantization) and the norm weights (fp16 values)."""

    def __init__(self, cfg, layers, final_norm, lm_head, embed):
        self.cfg = cfg                  # dict: d, n_heads, n_kv_heads, hd, ffn, vocab, eps, theta
        self.layers = layers            # list of dict: q, k, v, o, gate, up, down (fp16 bits [N,K]); attn_norm, ffn_norm
        self.final_norm = final_norm    # fp16 values [d]
        self.lm_head = lm_head          # fp16 bits [vocab, d]
        self.embed = embed              # fp16 values [vocab, d]


def dequantized(fmt, w):
    """The oracle's own quantization of fp32 W and its dequantized fp16 bits."""
    from .linear import quantize_and_pack
    _, s, z, codes = quantize_and_pack(fmt, w)
    return dequant_fp16(fmt, codes, s, z)


def lin(x16, w_bits):
    """A linear with fp16 inputs: the float64 product rounded to fp16 (the device's output type)."""
    return f16(linear_ref(fp16_bits(x16), w_bits))


def decode_step(model, tokens, pos, cache_k, cache_v):
    """One decode step for M sequences at position pos (all the same length).

    tokens [M] int; cache_k / cache_v: lists per layer of float64 arrays [M, S, n_kv_heads*hd]
    holding fp16 values, updated in place at position pos. Returns (logits fp16 values [M, vocab],
    next tokens [M], the residual stream after the last layer [M, d])."""
    c = model.cfg
    hd, H, Hkv = c["hd"], c["n_heads"], c["n_kv_heads"]
    x = np.asarray(model.embed, dtype=np.float64)[np.asarray(tokens)]
    for l, L in enumerate(model.layers):
        h = rmsnorm(x, L["attn_norm"], c["eps"])
        q, k, v = lin(h, L["q"]), lin(h, L["k"]), lin(h, L["v"])
        cache_k[l][:, pos, :] = f16(rope(k, pos, hd, c["theta"]))
        cache_v[l][:, pos, :] = v
        a = f16(attention(rope(q, pos, hd, c["theta"]), cache_k[l], cache_v[l], pos, H, Hkv, hd))
        x = x + lin(a, L["o"])
        h2 = rmsnorm(x, L["ffn_norm"], c["eps"])
        g, u = lin(h2, L["gate"]), lin(h2, L["up"])
        x = x + lin(silu_mul(g, u), L["down"])
    logits = lin(rmsnorm(x, model.final_norm, c["eps"]), model.lm_head)
    return logits, argmax_lowest(logits), x
