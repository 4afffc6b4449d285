"""Pins of the decode-step oracle (oracle/decode.py), and planted mistakes each pin must reject.

CPU only. The pins compare against hand-derived closed forms (tests/golden/decode_examples.txt),
exact facts (rotation by angle 0, preserved pair lengths, one cached position), scipy's softmax
and logistic function, and a model whose attention and feed-forward outputs are zero.
"""

import numpy as np

import oracle
from oracle import decode as D
from tests import pins


def test_pins_accept_the_oracle():
    assert pins.check_rmsnorm(D.rmsnorm)
    assert pins.check_rope(D.rope)
    assert pins.check_attention(D.attention)
    assert pins.check_silu_mul(D.silu_mul)
    assert pins.check_argmax(D.argmax_lowest)


# ---------------------------------------------------------------- planted mistakes
def test_rmsnorm_sum_instead_of_mean_is_caught():
    assert not pins.check_rmsnorm(lambda x, g, eps: D.f16(x / np.sqrt(np.sum(x * x, 1, keepdims=True) + eps) * g))


def test_rmsnorm_eps_outside_the_root_is_caught():
    assert not pins.check_rmsnorm(lambda x, g, eps: D.f16(x / (np.sqrt(np.mean(x * x, 1, keepdims=True)) + eps) * g))


def test_rope_rotate_half_pairing_is_caught():
    def bad(x, pos, hd, theta):   # pairs (i, i + hd/2) instead of (2i, 2i+1)
        m, w = x.shape
        h = x.reshape(m, w // hd, 2, hd // 2)
        a = D.rope_angles(pos, hd, theta)
        c, s = np.cos(a), np.sin(a)
        x0, x1 = h[:, :, 0], h[:, :, 1]
        return np.stack([x0 * c - x1 * s, x0 * s + x1 * c], axis=2).reshape(m, w)
    assert not pins.check_rope(bad)


def test_rope_frequency_exponent_is_caught():
    def bad(x, pos, hd, theta):   # theta^(-i/hd)
        m, w = x.shape
        h = x.reshape(m, w // hd, hd // 2, 2)
        a = pos * np.power(theta, -np.arange(hd // 2) / hd)
        c, s = np.cos(a), np.sin(a)
        out = np.stack([h[..., 0] * c - h[..., 1] * s, h[..., 0] * s + h[..., 1] * c], axis=-1)
        return out.reshape(m, w)
    assert not pins.check_rope(bad)


def test_rope_sign_of_sine_is_caught():
    assert not pins.check_rope(lambda x, pos, hd, theta: D.rope(x, -pos, hd, theta))


def test_attention_without_scale_is_caught():
    def bad(q, ck, cv, pos, H, Hkv, hd):
        return D.attention(q, ck, cv, pos, H, Hkv, hd) if hd == 1 else D.attention(q * np.sqrt(hd), ck, cv, pos, H, Hkv, hd)
    assert not pins.check_attention(bad)


def test_attention_excluding_the_current_position_is_caught():
    def bad(q, ck, cv, pos, H, Hkv, hd):
        return D.attention(q, ck, cv, max(pos - 1, 0), H, Hkv, hd)
    assert not pins.check_attention(bad)


def test_attention_head_mapping_is_caught():
    def bad(q, ck, cv, pos, H, Hkv, hd):   # kv head h % Hkv instead of h // (H / Hkv)
        out = np.zeros((q.shape[0], H * hd))
        for h in range(H):
            kv = h % Hkv
            sub = D.attention(q[:, h * hd:(h + 1) * hd], ck[:, :, kv * hd:(kv + 1) * hd], cv[:, :, kv * hd:(kv + 1) * hd],
                              pos, 1, 1, hd)
            out[:, h * hd:(h + 1) * hd] = sub
        return out
    assert not pins.check_attention(bad)


def test_silu_with_the_wrong_sign_is_caught():
    assert not pins.check_silu_mul(lambda g, u: D.f16(g / (1.0 + np.exp(g)) * u))


def test_argmax_ties_to_the_highest_index_are_caught():
    assert not pins.check_argmax(lambda x: (x.shape[1] - 1 - np.argmax(x[:, ::-1], axis=1)).astype(np.int32))


# ---------------------------------------------------------------- the whole step
def _tiny_model(zero_blocks):
    rng = np.random.default_rng(17)
    cfg = dict(d=64, n_heads=4, n_kv_heads=2, hd=16, ffn=96, vocab=50, eps=1e-5, theta=10000.0)
    d, hd, ffn, vocab = cfg["d"], cfg["hd"], cfg["ffn"], cfg["vocab"]
    f16b = lambda a: oracle.fp16_bits(a)
    layers = []
    for _ in range(2):
        w = lambda n, k: f16b(0.05 * rng.standard_normal((n, k)))
        L = dict(q=w(4 * hd, d), k=w(2 * hd, d), v=w(2 * hd, d), o=w(d, 4 * hd), gate=w(ffn, d), up=w(ffn, d),
                 down=w(d, ffn), attn_norm=D.f16(1 + 0.1 * rng.standard_normal(d)),
                 ffn_norm=D.f16(1 + 0.1 * rng.standard_normal(d)))
        if zero_blocks:
            L["o"] = np.zeros_like(L["o"])
            L["down"] = np.zeros_like(L["down"])
        layers.append(L)
    model = D.Model(cfg, layers, D.f16(1 + 0.1 * rng.standard_normal(d)), f16b(0.05 * rng.standard_normal((vocab, d))),
                    D.f16(rng.standard_normal((vocab, d))))
    return model


def test_step_with_zero_blocks_reduces_to_norm_and_output_layer():
    # o and down all zero: the residual stream stays the embedding, so the logits are the output
    # layer applied to the final norm of the embedding rows
    m = _tiny_model(True)
    c = m.cfg
    ck = [np.zeros((2, 8, 2 * c["hd"])) for _ in m.layers]
    cv = [np.zeros((2, 8, 2 * c["hd"])) for _ in m.layers]
    tokens = np.array([3, 41])
    logits, nxt, x = D.decode_step(m, tokens, 5, ck, cv)
    e = m.embed[tokens]
    assert np.array_equal(x, e)
    h = D.rmsnorm(e, m.final_norm, c["eps"])
    want = D.f16(oracle.fp16_from_bits(oracle.fp16_bits(h)) @ oracle.fp16_from_bits(m.lm_head).T)
    assert np.array_equal(logits, want)
    assert np.array_equal(nxt, np.argmax(want, axis=1))
    # the step wrote position 5 of every cache and nothing else
    for a in ck + cv:
        assert np.any(a[:, 5] != 0) and not np.any(a[:, :5]) and not np.any(a[:, 6:])


def test_step_cache_holds_rotated_keys_and_plain_values():
    m = _tiny_model(False)
    c = m.cfg
    ck = [np.zeros((1, 8, 2 * c["hd"])) for _ in m.layers]
    cv = [np.zeros((1, 8, 2 * c["hd"])) for _ in m.layers]
    D.decode_step(m, np.array([7]), 3, ck, cv)
    h = D.rmsnorm(m.embed[[7]], m.layers[0]["attn_norm"], c["eps"])
    k = D.lin(h, m.layers[0]["k"])
    v = D.lin(h, m.layers[0]["v"])
    assert np.array_equal(cv[0][:, 3], v)
    assert np.array_equal(ck[0][:, 3], D.f16(D.rope(k, 3, c["hd"], c["theta"])))
