"""Pins of the prefix-producer oracle (oracle/prefix.py) against things other
than itself: torch's float64 library routines (rms_norm, scaled-dot-product
attention, tanh GELU), a complex-number form of the rotary encoding, closed
forms when the residual branches are switched off, and invariants (the
last layer's attention and MLP reach no output; samples are independent;
attention is bidirectional over the prefix)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import prefix as PO
from synth import PREFIX_CONFIGS, make_prefix_inputs, prefix_param_specs


def micro(**kw):
    base = dict(name="micro_prefix", num_layers=2, width=16, num_q_heads=4, num_kv_heads=2, head_dim=8,
                mlp_dim=24, prefix_len=7, batch=2, seed=21, weight_std=0.3)
    base.update(kw)
    return PREFIX_CONFIGS["prefix_tiny"].replace(**base)


def f64(params):
    return {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}


def t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def rope_complex(x, pos, base):
    """Rotary encoding written with complex numbers: pair (j, j + d/2) is the
    complex value x_j + i x_{j+d/2}, multiplied by exp(i pos base^(-2j/d))."""
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    theta = np.array([base ** (-2.0 * j / d) for j in range(half)])
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def kv_closed_form(p, l, x, cfg):
    """K and V of layer l for residual stream x [B, P, W], per token, with
    torch's rms_norm and the complex rotary form."""
    B, P, W = x.shape
    Hkv, d = cfg.num_kv_heads, cfg.head_dim
    xn = F.rms_norm(t(x), (W,), weight=1.0 + t(p[f"layers.{l}.attn_norm.w"]), eps=cfg.rms_eps).numpy()
    k = (xn @ p[f"layers.{l}.k.w"]).reshape(B, P, Hkv, d)
    v = (xn @ p[f"layers.{l}.v.w"]).reshape(B, P, Hkv, d)
    for b in range(B):
        for h in range(Hkv):
            k[b, :, h] = rope_complex(k[b, :, h], np.arange(P), cfg.rope_base)
    return k, v


def torch_layer(p, l, x, cfg):
    """One full decoder layer with torch library routines (float64)."""
    B, P, W = x.shape
    Hq, Hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    X = t(x)
    xn = F.rms_norm(X, (W,), weight=1.0 + t(p[f"layers.{l}.attn_norm.w"]), eps=cfg.rms_eps)
    q = (xn @ t(p[f"layers.{l}.q.w"])).reshape(B, P, Hq, d).numpy()
    k, v = kv_closed_form(p, l, x, cfg)
    for b in range(B):
        for h in range(Hq):
            q[b, :, h] = rope_complex(q[b, :, h], np.arange(P), cfg.rope_base)
    Q = t(q).transpose(1, 2)
    K = t(k).transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    V = t(v).transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    o = F.scaled_dot_product_attention(Q, K, V, is_causal=False).transpose(1, 2).reshape(B, P, Hq * d)
    X = X + o @ t(p[f"layers.{l}.o.w"])
    xn = F.rms_norm(X, (W,), weight=1.0 + t(p[f"layers.{l}.mlp_norm.w"]), eps=cfg.rms_eps)
    a = F.gelu(xn @ t(p[f"layers.{l}.gate.w"]), approximate="tanh") * (xn @ t(p[f"layers.{l}.up.w"]))
    return (X + a @ t(p[f"layers.{l}.down.w"])).numpy()


def test_gain_rms_norm_vs_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32)) * 3.0
    w = rng.standard_normal(32) * 0.5
    want = F.rms_norm(t(x), (32,), weight=1.0 + t(w), eps=1e-6).numpy()
    np.testing.assert_allclose(PO.gain_rms_norm(x, w, 1e-6), want, rtol=1e-13, atol=0)
    # a zero gain weight is a plain RMS normalisation: unit mean square
    y = PO.gain_rms_norm(x, np.zeros(32), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)


def test_first_layer_kv_closed_form():
    cfg = micro()
    params, emb = make_prefix_inputs(cfg)
    p = f64(params)
    pk, pv = PO.prefix_kv(params, emb, cfg)
    assert pk.shape == (cfg.num_layers, cfg.batch, cfg.prefix_len, cfg.num_kv_heads, cfg.head_dim)
    k, v = kv_closed_form(p, 0, emb.astype(np.float64), cfg)
    np.testing.assert_allclose(pk[0], k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(pv[0], v, rtol=0, atol=1e-12)


def test_zero_branches_keep_the_stream():
    """With every o and down projection zero the residual stream stays the
    embeddings, so every layer's K/V is the closed form of its own weights on
    the embeddings: a wrong layer index or norm weight fails."""
    cfg = micro(num_layers=3)
    params, emb = make_prefix_inputs(cfg)
    for l in range(cfg.num_layers):
        params[f"layers.{l}.o.w"][:] = 0.0
        params[f"layers.{l}.down.w"][:] = 0.0
    p = f64(params)
    pk, pv = PO.prefix_kv(params, emb, cfg)
    for l in range(cfg.num_layers):
        k, v = kv_closed_form(p, l, emb.astype(np.float64), cfg)
        np.testing.assert_allclose(pk[l], k, rtol=0, atol=1e-12)
        np.testing.assert_allclose(pv[l], v, rtol=0, atol=1e-12)


def test_second_layer_vs_torch_layer():
    """Layer 1's K/V is the closed form on the stream that a full torch layer
    (rms_norm, bidirectional sdpa, tanh GELU) makes from the embeddings."""
    cfg = micro()
    params, emb = make_prefix_inputs(cfg)
    p = f64(params)
    pk, pv = PO.prefix_kv(params, emb, cfg)
    x1 = torch_layer(p, 0, emb.astype(np.float64), cfg)
    k, v = kv_closed_form(p, 1, x1, cfg)
    np.testing.assert_allclose(pk[1], k, rtol=0, atol=1e-11)
    np.testing.assert_allclose(pv[1], v, rtol=0, atol=1e-11)


def test_attention_is_bidirectional():
    """The first token's layer-1 keys depend on the last token's embedding."""
    cfg = micro(batch=1)
    params, emb = make_prefix_inputs(cfg)
    pk, _ = PO.prefix_kv(params, emb, cfg)
    emb2 = emb.copy()
    emb2[0, -1] += 1.0
    pk2, _ = PO.prefix_kv(params, emb2, cfg)
    assert np.array_equal(pk[0, 0, 0], pk2[0, 0, 0])          # layer 0 is per token
    assert np.abs(pk[1, 0, 0] - pk2[1, 0, 0]).max() > 1e-6


def test_last_layer_attention_and_mlp_reach_no_output():
    cfg = micro()
    params, emb = make_prefix_inputs(cfg)
    pk, pv = PO.prefix_kv(params, emb, cfg)
    last = cfg.num_layers - 1
    for n in ("q", "o", "gate", "up", "down"):
        params[f"layers.{last}.{n}.w"] = params[f"layers.{last}.{n}.w"] * 3.0 + 1.0
    params[f"layers.{last}.mlp_norm.w"] = params[f"layers.{last}.mlp_norm.w"] + 5.0
    pk2, pv2 = PO.prefix_kv(params, emb, cfg)
    assert np.array_equal(pk, pk2) and np.array_equal(pv, pv2)


def test_samples_are_independent():
    cfg = micro(batch=3)
    params, emb = make_prefix_inputs(cfg)
    pk, pv = PO.prefix_kv(params, emb, cfg)
    one = cfg.replace(batch=1)
    for b in range(3):
        k1, v1 = PO.prefix_kv(params, emb[b:b + 1], one)
        np.testing.assert_allclose(pk[:, b:b + 1], k1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(pv[:, b:b + 1], v1, rtol=0, atol=1e-13)


def test_prefix_workload_shapes():
    cfg = PREFIX_CONFIGS["prefix_gemma2b_p560"]
    specs = dict(prefix_param_specs(cfg))
    assert specs["layers.0.q.w"] == (2048, 2048) and specs["layers.0.k.w"] == (2048, 256)
    assert specs["layers.17.gate.w"] == (2048, 16384) and specs["layers.17.down.w"] == (16384, 2048)
    n = sum(int(np.prod(s)) for s in specs.values())
    assert 1.9e9 < n < 2.1e9          # the decoder of a ~2B-parameter VLM (embedding table excluded)
