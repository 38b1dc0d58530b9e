"""Pins of the pi0 oracle (oracle/pi0.py): torch library routines for the
action-time MLP and for a masked attention block, closed forms when
branches are switched off, the mask's invariant (the state token never sees
the action tokens) and the Euler loop's constant-velocity closed form."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import denoise as O
from oracle import pi0 as P0
from synth import CONFIGS, make_inputs


def micro(**kw):
    base = dict(name="micro_pi0", num_layers=2, width=8, num_q_heads=2, num_kv_heads=1, head_dim=4, mlp_dim=12,
                action_horizon=3, action_dim=3, state_dim=2, time_emb_dim=8, prefix_len=4, batch=2, num_steps=2,
                seed=31, weight_std=0.3)
    base.update(kw)
    return CONFIGS["pi0_tiny_fp32"].replace(**base)


def f64(params):
    return {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}


def t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def test_action_time_input_vs_torch():
    cfg = micro()
    params, _, _, noise, _ = make_inputs(cfg)
    p = f64(params)
    a = t(noise) @ t(p["in_proj.w"]) + t(p["in_proj.b"])
    half = cfg.width // 2
    frac = torch.arange(half, dtype=torch.float64) / (half - 1)
    period = 4e-3 * (4.0 / 4e-3) ** frac
    tt = 0.7
    e = torch.cat([torch.sin(2 * math.pi * tt / period), torch.cos(2 * math.pi * tt / period)])
    cat = torch.cat([a, e.expand(a.shape[0], a.shape[1], -1)], dim=-1)
    u = F.silu(F.linear(cat, t(p["time_mlp_in.w"]).T, t(p["time_mlp_in.b"])))
    want = F.linear(u, t(p["time_mlp_out.w"]).T, t(p["time_mlp_out.b"])).numpy()
    np.testing.assert_allclose(P0.action_time_input(p, noise.astype(np.float64), tt), want, rtol=1e-12, atol=1e-13)


def test_layer_vs_torch_with_boolean_mask():
    """One block against torch rms_norm + sdpa with an explicit boolean mask
    (state query row sees prefix and itself) + tanh GELU."""
    cfg = micro()
    params, pk, pv, noise, state = make_inputs(cfg)
    p = f64(params)
    rng = np.random.default_rng(5)
    B, T, W, Pn = cfg.batch, cfg.action_horizon + 1, cfg.width, cfg.prefix_len
    Hq, Hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    h = rng.standard_normal((B, T, W))
    got = P0.pi0_layer(p, 0, h, pk[0].astype(np.float64), pv[0].astype(np.float64), cfg)
    H = t(h)
    xn = F.rms_norm(H, (W,), weight=1.0 + t(p["layers.0.attn_norm.w"]), eps=cfg.rms_eps)
    pos = np.arange(Pn, Pn + T)
    q = O.rope((xn @ t(p["layers.0.q.w"])).reshape(B, T, Hq, d).permute(0, 2, 1, 3).numpy(), pos, cfg.rope_base)
    k = O.rope((xn @ t(p["layers.0.k.w"])).reshape(B, T, Hkv, d).permute(0, 2, 1, 3).numpy(), pos, cfg.rope_base)
    v = (xn @ t(p["layers.0.v.w"])).reshape(B, T, Hkv, d).permute(0, 2, 1, 3)
    K = torch.cat([t(pk[0]).permute(0, 2, 1, 3), t(k)], dim=2).repeat_interleave(Hq // Hkv, dim=1)
    V = torch.cat([t(pv[0]).permute(0, 2, 1, 3), v], dim=2).repeat_interleave(Hq // Hkv, dim=1)
    mask = torch.ones(T, Pn + T, dtype=torch.bool)
    mask[0, Pn + 1:] = False
    o = F.scaled_dot_product_attention(t(q), K, V, attn_mask=mask).permute(0, 2, 1, 3).reshape(B, T, Hq * d)
    H = H + o @ t(p["layers.0.o.w"])
    xn = F.rms_norm(H, (W,), weight=1.0 + t(p["layers.0.mlp_norm.w"]), eps=cfg.rms_eps)
    want = H + (F.gelu(xn @ t(p["layers.0.gate.w"]), approximate="tanh") * (xn @ t(p["layers.0.up.w"]))) @ t(p["layers.0.down.w"])
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-12)


def test_state_token_never_sees_the_actions():
    cfg = micro()
    params, pk, pv, _, _ = make_inputs(cfg)
    p = f64(params)
    rng = np.random.default_rng(6)
    h = rng.standard_normal((cfg.batch, cfg.action_horizon + 1, cfg.width))
    h2 = h.copy()
    h2[:, 1:] += rng.standard_normal(h2[:, 1:].shape)
    a = P0.pi0_layer(p, 0, h, pk[0].astype(np.float64), pv[0].astype(np.float64), cfg)
    b = P0.pi0_layer(p, 0, h2, pk[0].astype(np.float64), pv[0].astype(np.float64), cfg)
    np.testing.assert_array_equal(a[:, 0], b[:, 0])
    assert np.abs(a[:, 1:] - b[:, 1:]).max() > 1e-3
    # and the actions do see the state token
    h3 = h.copy()
    h3[:, 0] += 1.0
    c = P0.pi0_layer(p, 0, h3, pk[0].astype(np.float64), pv[0].astype(np.float64), cfg)
    assert np.abs(c[:, 1:] - a[:, 1:]).max() > 1e-6


def test_zero_layers_closed_form():
    """L = 0: v = norm(action-time input) (1 + w_f) W_out + b_out, whatever the state."""
    cfg = micro(num_layers=0)
    params, pk, pv, noise, state = make_inputs(cfg)
    p = f64(params)
    x = noise.astype(np.float64)
    s = state.astype(np.float64) @ p["state_proj.w"] + p["state_proj.b"]
    got = P0.velocity_pi0(p, x, s, 0.3, pk, pv, cfg)
    a = P0.action_time_input(p, x, 0.3)
    want = F.rms_norm(t(a), (cfg.width,), weight=1.0 + t(p["final_norm.w"]), eps=cfg.rms_eps).numpy() @ p["out_proj.w"] + p["out_proj.b"]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    got2 = P0.velocity_pi0(p, x, s * 7.0, 0.3, pk, pv, cfg)
    np.testing.assert_array_equal(got, got2)


def test_constant_velocity_and_zero_out_projection():
    cfg = micro()
    params, pk, pv, noise, state = make_inputs(cfg)
    params["out_proj.w"][:] = 0.0
    x0 = P0.denoise_pi0(params, noise, state, pk, pv, cfg)
    np.testing.assert_allclose(x0, noise.astype(np.float64) - params["out_proj.b"].astype(np.float64), rtol=0, atol=1e-12)
    params["out_proj.b"][:] = 0.0
    x0 = P0.denoise_pi0(params, noise, state, pk, pv, cfg)
    np.testing.assert_array_equal(x0, noise.astype(np.float64))


def test_single_step_is_one_velocity_call():
    cfg = micro(num_steps=1)
    params, pk, pv, noise, state = make_inputs(cfg)
    p = f64(params)
    s = state.astype(np.float64) @ p["state_proj.w"] + p["state_proj.b"]
    v = P0.velocity_pi0(p, noise.astype(np.float64), s, 1.0, pk.astype(np.float64), pv.astype(np.float64), cfg)
    np.testing.assert_allclose(P0.denoise_pi0(params, noise, state, pk, pv, cfg), noise - v, rtol=0, atol=1e-13)


def test_samples_are_independent():
    cfg = micro(batch=3)
    params, pk, pv, noise, state = make_inputs(cfg)
    full = P0.denoise_pi0(params, noise, state, pk, pv, cfg)
    one = cfg.replace(batch=1)
    for b in range(3):
        x = P0.denoise_pi0(params, noise[b:b + 1], state[b:b + 1], pk[:, b:b + 1], pv[:, b:b + 1], one)
        np.testing.assert_allclose(full[b:b + 1], x, rtol=0, atol=1e-13)
