"""Pins of the CPU oracle against things other than itself: brute force on tiny
inputs, closed forms, invariants, special cases that reduce to library
routines. Each check is chosen so that a plausible slip in the oracle (a
dropped term, a sign, a transposed operand, a wrong index) fails it."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import denoise as O
from synth import CONFIGS, make_inputs

RNG = np.random.default_rng(1234)


def micro_cfg(**kw):
    base = dict(name="micro", num_layers=1, width=8, num_q_heads=2, num_kv_heads=1, head_dim=4,
                mlp_dim=16, action_horizon=2, action_dim=3, state_dim=2, time_emb_dim=8,
                prefix_len=3, batch=1, num_steps=2, weight_precision="fp32", seed=7, weight_std=0.3)
    base.update(kw)
    return CONFIGS["tiny_fp32"].replace(**base)


# ----------------------------------------------------------------------------- attention
def brute_attention(q, k, v):
    """Triple loop, math.exp, no vectorisation. q [B,Hq,T,d], k/v [B,Hkv,S,d]."""
    B, Hq, T, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            for t in range(T):
                logits = []
                for s in range(S):
                    acc = 0.0
                    for j in range(d):
                        acc += q[b, h, t, j] * k[b, kh, s, j]
                    logits.append(acc / math.sqrt(d))
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                z = sum(w)
                for j in range(d):
                    out[b, h, t, j] = sum(w[s] * v[b, kh, s, j] for s in range(S)) / z
    return out


def test_attention_brute_force():
    q = RNG.standard_normal((2, 4, 3, 4))
    k = RNG.standard_normal((2, 2, 5, 4))
    v = RNG.standard_normal((2, 2, 5, 4))
    np.testing.assert_allclose(O.gqa_attention(q, k, v), brute_attention(q, k, v), rtol=0, atol=1e-12)


def test_attention_vs_torch_sdpa():
    q = RNG.standard_normal((1, 8, 6, 16))
    k = RNG.standard_normal((1, 1, 11, 16))
    v = RNG.standard_normal((1, 1, 11, 16))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         enable_gqa=True).numpy()
    np.testing.assert_allclose(O.gqa_attention(q, k, v), ref, rtol=0, atol=1e-12)


def test_attention_special_cases():
    q = RNG.standard_normal((1, 2, 3, 4))
    v1 = RNG.standard_normal((1, 1, 1, 4))
    k1 = RNG.standard_normal((1, 1, 1, 4))
    # a single key returns its value
    np.testing.assert_allclose(O.gqa_attention(q, k1, v1), np.broadcast_to(v1, (1, 2, 3, 4)), atol=1e-15)
    # equal keys: uniform weights -> mean of V
    k = np.repeat(k1, 5, axis=2)
    v = RNG.standard_normal((1, 1, 5, 4))
    np.testing.assert_allclose(O.gqa_attention(q, k, v), np.broadcast_to(v.mean(axis=2, keepdims=True), (1, 2, 3, 4)),
                               atol=1e-14)
    # one KV head shared by all query heads == MHA with replicated KV
    k = RNG.standard_normal((1, 1, 5, 4))
    rep = O.gqa_attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1))
    np.testing.assert_allclose(O.gqa_attention(q, k, v), rep, atol=1e-15)
    # a key far ahead of the others takes all the weight
    k2 = k.copy()
    k2[0, 0, 2] = 50.0 * q[0, 0, 0] / np.linalg.norm(q[0, 0, 0])
    o = O.gqa_attention(q[:, :1, :1], k2, v)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 2], atol=1e-10)


# ----------------------------------------------------------------------------- norms, rope, gelu, embedding
def test_rms_norm_vs_torch():
    h = RNG.standard_normal((3, 5, 32)) * 3.0
    ref = F.rms_norm(torch.from_numpy(h), (32,), eps=1e-6).numpy()
    zero = np.zeros(32)
    np.testing.assert_allclose(O.ada_rms_norm(h, zero, zero, 1e-6), ref, atol=1e-13)


def test_ada_rms_norm_invariants():
    h = RNG.standard_normal((4, 16))
    sc, sh = RNG.standard_normal(16), RNG.standard_normal(16)
    # positive scaling invariance (eps -> 0)
    np.testing.assert_allclose(O.ada_rms_norm(7.5 * h, sc, sh, 0.0), O.ada_rms_norm(h, sc, sh, 0.0), atol=1e-13)
    # zero modulation -> unit RMS
    y = O.ada_rms_norm(h, 0 * sc, 0 * sh, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)
    # scale and shift act per feature: y = n * (1 + sc) + sh
    n = O.ada_rms_norm(h, 0 * sc, 0 * sh, 0.0)
    np.testing.assert_allclose(O.ada_rms_norm(h, sc, sh, 0.0), n + n * sc + sh, atol=1e-13)


def test_rope_properties():
    d = 8
    x = RNG.standard_normal((2, 5, d))
    np.testing.assert_allclose(O.rope(x, np.zeros(5), 10000.0), x, atol=0)
    y = O.rope(x, np.arange(3, 8), 10000.0)
    # each (j, j + d/2) pair keeps its norm
    np.testing.assert_allclose(x[..., :4] ** 2 + x[..., 4:] ** 2, y[..., :4] ** 2 + y[..., 4:] ** 2, atol=1e-13)
    # <R_m q, R_n k> depends only on m - n
    q = RNG.standard_normal((1, d))
    k = RNG.standard_normal((1, d))
    a = O.rope(q, [5], 100.0) @ O.rope(k, [2], 100.0).T
    b = O.rope(q, [13], 100.0) @ O.rope(k, [10], 100.0).T
    np.testing.assert_allclose(a, b, atol=1e-12)
    # the rotation direction: position 1, pair 0 rotates by angle 1 (inv_freq_0 = 1)
    e = np.zeros((1, d)); e[0, 0] = 1.0
    r = O.rope(e, [1], 10000.0)
    np.testing.assert_allclose([r[0, 0], r[0, 4]], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    # the highest pair turns by base^(-2(d/2-1)/d) radians per position
    e = np.zeros((1, d)); e[0, 3] = 1.0
    r = O.rope(e, [1], 10000.0)
    ang = 10000.0 ** (-2.0 * 3 / d)
    np.testing.assert_allclose([r[0, 3], r[0, 7]], [math.cos(ang), math.sin(ang)], atol=1e-15)


def test_gelu_and_silu():
    u = np.linspace(-6, 6, 101)
    ref = F.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(u), ref, atol=1e-14)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.gelu_tanh(u) - O.gelu_tanh(-u), u, atol=1e-14)
    np.testing.assert_allclose(O.silu(u), F.silu(torch.from_numpy(u)).numpy(), atol=1e-14)


def test_sincos_embedding():
    for t in (0.0, 0.1, 0.37, 1.0):
        e = O.sincos_embedding(t, 16)
        np.testing.assert_allclose(e[:8] ** 2 + e[8:] ** 2, 1.0, atol=1e-15)
    e0 = O.sincos_embedding(0.0, 16)
    assert np.all(e0[:8] == 0.0) and np.all(e0[8:] == 1.0)
    # first period is 4e-3, last is 4.0
    e = O.sincos_embedding(1e-3, 16)
    np.testing.assert_allclose(e[0], math.sin(2 * math.pi * 1e-3 / 4e-3), atol=1e-15)
    np.testing.assert_allclose(e[7], math.sin(2 * math.pi * 1e-3 / 4.0), atol=1e-15)


# ----------------------------------------------------------------------------- Euler loop closed forms
def _set_const_velocity(params, vel):
    p = dict(params)
    p["out_proj.w"] = np.zeros_like(p["out_proj.w"])
    p["out_proj.b"] = np.asarray(vel, dtype=np.float32)
    return p


def test_constant_velocity_closed_form():
    cfg = CONFIGS["tiny_fp32"]
    params, pk, pv, noise, state = make_inputs(cfg)
    vel = RNG.standard_normal(cfg.action_dim).astype(np.float32)
    x0 = O.denoise(_set_const_velocity(params, vel), noise, state, pk, pv, cfg)
    np.testing.assert_allclose(x0, noise.astype(np.float64) - vel.astype(np.float64), atol=1e-14, rtol=0)


def test_zero_out_projection_is_identity_bitwise():
    cfg = CONFIGS["tiny_fp32"]
    params, pk, pv, noise, state = make_inputs(cfg)
    x0 = O.denoise(_set_const_velocity(params, np.zeros(cfg.action_dim)), noise, state, pk, pv, cfg)
    assert np.array_equal(x0, noise.astype(np.float64))


def test_single_step_is_one_euler_step():
    cfg = micro_cfg(num_layers=1)
    params, pk, pv, noise, state = make_inputs(cfg)
    p = O.to_f64(params)
    s = state.astype(np.float64) @ p["state_proj.w"] + p["state_proj.b"]
    v = O.velocity(p, noise.astype(np.float64), s, 1.0, pk.astype(np.float64), pv.astype(np.float64), cfg)
    x1 = O.denoise(params, noise, state, pk, pv, cfg, num_steps=1)
    np.testing.assert_allclose(x1, noise - v, atol=1e-15)


def test_time_grid_and_step_sign():
    """Zero input projections make h = 0, so the zero-layer velocity is
    shift_final(t) @ W_out + b_out: the loop must sum dt * v(t_k) over
    t_k = (N-k)/N with dt = -1/N."""
    cfg = micro_cfg(num_layers=0)
    params, pk, pv, noise, state = make_inputs(cfg)
    for n in ("in_proj.w", "in_proj.b", "state_proj.w", "state_proj.b"):
        params[n] = np.zeros_like(params[n])
    p = O.to_f64(params)
    N, W = 4, cfg.width
    x = noise.astype(np.float64)
    for k in range(N):
        c = O.time_conditioning(p, (N - k) / N)
        shift = (c @ p["final_norm.mod.w"] + p["final_norm.mod.b"])[W:2 * W]
        x = x - (shift @ p["out_proj.w"] + p["out_proj.b"]) / N
    np.testing.assert_allclose(O.denoise(params, noise, state, pk, pv, cfg, num_steps=N), x, atol=1e-15)


def test_zero_layer_closed_form():
    """L = 0: v = adanorm_final(x W_in + b_in + s) W_out + b_out, written out directly."""
    cfg = micro_cfg(num_layers=0, width=6, action_dim=3, state_dim=2, time_emb_dim=4)
    params, pk, pv, noise, state = make_inputs(cfg)
    p = {k: v.astype(np.float64) for k, v in params.items()}
    x = noise.astype(np.float64)[0]                   # [H, A]
    N = 2
    for k in range(N):
        t = (N - k) / N
        e = np.array([math.sin(2 * math.pi * t / 4e-3), math.sin(2 * math.pi * t / 4.0),
                      math.cos(2 * math.pi * t / 4e-3), math.cos(2 * math.pi * t / 4.0)])
        h1 = e @ p["time_mlp_in.w"] + p["time_mlp_in.b"]
        h1 = h1 / (1 + np.exp(-h1))
        c = h1 @ p["time_mlp_out.w"] + p["time_mlp_out.b"]
        c = c / (1 + np.exp(-c))
        m = c @ p["final_norm.mod.w"] + p["final_norm.mod.b"]
        sc, sh = m[:6], m[6:12]
        s = state[0].astype(np.float64) @ p["state_proj.w"] + p["state_proj.b"]
        h = x @ p["in_proj.w"] + p["in_proj.b"] + s
        y = np.empty_like(h)
        for i in range(h.shape[0]):
            r = math.sqrt(sum(hh * hh for hh in h[i]) / 6 + cfg.rms_eps)
            y[i] = h[i] / r * (1 + sc) + sh
        v = y @ p["out_proj.w"] + p["out_proj.b"]
        x = x - v / N
    np.testing.assert_allclose(O.denoise(params, noise, state, pk, pv, cfg), x[None], atol=1e-13)


# ----------------------------------------------------------------------------- micro brute force of a whole step
def brute_velocity(p, cfg, x, s, t, pk, pv):
    """Pure-Python loops over every index; x [H][A], s [W], pk/pv [L][P][Hkv][d] (batch 1)."""
    W, Hq, Hkv, d, Fd = cfg.width, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.mlp_dim
    T, A, E, P = cfg.action_horizon, cfg.action_dim, cfg.time_emb_dim, cfg.prefix_len
    eps = cfg.rms_eps

    def mat(vec, w, b=None):
        n_out = w.shape[1]
        out = [sum(vec[i] * w[i][j] for i in range(len(vec))) for j in range(n_out)]
        if b is not None:
            out = [out[j] + b[j] for j in range(n_out)]
        return out

    def sig(z):
        return z / (1.0 + math.exp(-z))

    half = E // 2
    e = [0.0] * E
    for i in range(half):
        per = 4e-3 * (4.0 / 4e-3) ** (i / (half - 1))
        e[i] = math.sin(2 * math.pi * t / per)
        e[half + i] = math.cos(2 * math.pi * t / per)
    c = [sig(z) for z in mat(e, p["time_mlp_in.w"], p["time_mlp_in.b"])]
    c = [sig(z) for z in mat(c, p["time_mlp_out.w"], p["time_mlp_out.b"])]

    def mod(name):
        m = mat(c, p[name + ".w"], p[name + ".b"])
        return m[:W], m[W:2 * W], m[2 * W:]

    def anorm(row, sc, sh):
        r = math.sqrt(sum(z * z for z in row) / W + eps)
        return [row[j] / r * (1 + sc[j]) + sh[j] for j in range(W)]

    def rot(vec, pos):
        out = list(vec)
        for j in range(d // 2):
            ang = pos * cfg.rope_base ** (-2.0 * j / d)
            a, b = vec[j], vec[j + d // 2]
            out[j] = a * math.cos(ang) - b * math.sin(ang)
            out[j + d // 2] = b * math.cos(ang) + a * math.sin(ang)
        return out

    h = [[v + s[j] for j, v in enumerate(mat(x[i], p["in_proj.w"], p["in_proj.b"]))] for i in range(T)]
    for l in range(cfg.num_layers):
        pre = f"layers.{l}."
        sc, sh, g = mod(pre + "attn_norm.mod")
        xn = [anorm(h[i], sc, sh) for i in range(T)]
        q = [mat(xn[i], p[pre + "q.w"]) for i in range(T)]
        k = [mat(xn[i], p[pre + "k.w"]) for i in range(T)]
        v = [mat(xn[i], p[pre + "v.w"]) for i in range(T)]
        o = [[0.0] * (Hq * d) for _ in range(T)]
        for i in range(T):
            for hh in range(Hq):
                kh = hh // (Hq // Hkv)
                qi = rot(q[i][hh * d:(hh + 1) * d], P + i)
                keys = [list(pk[l][j][kh]) for j in range(P)] + [rot(k[j][kh * d:(kh + 1) * d], P + j) for j in range(T)]
                vals = [list(pv[l][j][kh]) for j in range(P)] + [v[j][kh * d:(kh + 1) * d] for j in range(T)]
                lg = [sum(qi[z] * kk[z] for z in range(d)) / math.sqrt(d) for kk in keys]
                mx = max(lg)
                wts = [math.exp(z - mx) for z in lg]
                tot = sum(wts)
                for z in range(d):
                    o[i][hh * d + z] = sum(wts[j] * vals[j][z] for j in range(len(keys))) / tot
        h = [[h[i][j] + g[j] * y for j, y in enumerate(mat(o[i], p[pre + "o.w"]))] for i in range(T)]
        sc, sh, g = mod(pre + "mlp_norm.mod")
        xn = [anorm(h[i], sc, sh) for i in range(T)]
        for i in range(T):
            gt = mat(xn[i], p[pre + "gate.w"])
            up = mat(xn[i], p[pre + "up.w"])
            a = [0.5 * gt[j] * (1 + math.tanh(math.sqrt(2 / math.pi) * (gt[j] + 0.044715 * gt[j] ** 3))) * up[j]
                 for j in range(Fd)]
            dn = mat(a, p[pre + "down.w"])
            h[i] = [h[i][j] + g[j] * dn[j] for j in range(W)]
    sc, sh, _ = mod("final_norm.mod")
    return [mat(anorm(h[i], sc, sh), p["out_proj.w"], p["out_proj.b"]) for i in range(T)]


@pytest.mark.parametrize("layers", [1, 2])
def test_micro_brute_force_denoise(layers):
    cfg = micro_cfg(num_layers=layers)
    params, pk, pv, noise, state = make_inputs(cfg)
    p = {k: v.astype(np.float64) for k, v in params.items()}
    x = noise[0].astype(np.float64).tolist()
    s = (state[0].astype(np.float64) @ p["state_proj.w"] + p["state_proj.b"]).tolist()
    N = cfg.num_steps
    for k in range(N):
        v = brute_velocity(p, cfg, x, s, (N - k) / N, pk[:, 0].astype(np.float64), pv[:, 0].astype(np.float64))
        x = [[x[i][j] - v[i][j] / N for j in range(cfg.action_dim)] for i in range(cfg.action_horizon)]
    np.testing.assert_allclose(O.denoise(params, noise, state, pk, pv, cfg), np.array(x)[None], atol=1e-12, rtol=0)


def test_micro_brute_force_batch_independent():
    """Samples of a batch never mix: batch-2 run == two batch-1 runs."""
    cfg = micro_cfg(num_layers=1, batch=2)
    params, pk, pv, noise, state = make_inputs(cfg)
    out = O.denoise(params, noise, state, pk, pv, cfg)
    for b in range(2):
        c1 = cfg.replace(batch=1)
        one = O.denoise(params, noise[b:b + 1], state[b:b + 1], pk[:, b:b + 1], pv[:, b:b + 1], c1)
        np.testing.assert_allclose(out[b:b + 1], one, atol=1e-15)


# ----------------------------------------------------------------------------- plain pre-norm block via torch
def test_plain_block_special_case_vs_torch():
    """gate = 1, scale = shift = 0 reduces a layer to a plain pre-norm block,
    which is rebuilt here from torch's rms_norm / SDPA / gelu routines."""
    cfg = micro_cfg(num_layers=1, width=16, num_q_heads=4, num_kv_heads=2, head_dim=8, mlp_dim=32,
                    action_horizon=5, prefix_len=7, batch=2, weight_std=0.2)
    params, pk, pv, noise, state = make_inputs(cfg)
    p = {k: v.astype(np.float64) for k, v in params.items()}
    W = cfg.width
    for n in ("layers.0.attn_norm.mod", "layers.0.mlp_norm.mod"):
        p[n + ".w"] = np.zeros_like(p[n + ".w"])
        b = np.zeros(3 * W); b[2 * W:] = 1.0
        p[n + ".b"] = b
    h = RNG.standard_normal((2, 5, W))
    c = RNG.standard_normal(W)
    got = O.expert_layer(p, 0, h, c, pk[0].astype(np.float64), pv[0].astype(np.float64), cfg)

    T = torch.from_numpy
    ht = T(h)
    d, Hq, Hkv = 8, 4, 2
    xn = F.rms_norm(ht, (W,), eps=cfg.rms_eps)
    q = (xn @ T(p["layers.0.q.w"])).view(2, 5, Hq, d).transpose(1, 2)
    k = (xn @ T(p["layers.0.k.w"])).view(2, 5, Hkv, d).transpose(1, 2)
    v = (xn @ T(p["layers.0.v.w"])).view(2, 5, Hkv, d).transpose(1, 2)
    pos = torch.arange(7, 12, dtype=torch.float64)
    inv = cfg.rope_base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = pos[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)
    sin = torch.cat([ang.sin(), ang.sin()], -1)

    def rot_half(x):
        return torch.cat([-x[..., d // 2:], x[..., :d // 2]], -1)

    q = q * cos + rot_half(q) * sin
    k = k * cos + rot_half(k) * sin
    K = torch.cat([T(pk[0]).double().transpose(1, 2), k], 2)
    V = torch.cat([T(pv[0]).double().transpose(1, 2), v], 2)
    o = F.scaled_dot_product_attention(q, K, V, enable_gqa=True).transpose(1, 2).reshape(2, 5, Hq * d)
    ht = ht + o @ T(p["layers.0.o.w"])
    xn = F.rms_norm(ht, (W,), eps=cfg.rms_eps)
    a = F.gelu(xn @ T(p["layers.0.gate.w"]), approximate="tanh") * (xn @ T(p["layers.0.up.w"]))
    ref = (ht + a @ T(p["layers.0.down.w"])).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_modulation_table_matches_per_step_conditioning():
    cfg = micro_cfg(num_layers=2)
    params, *_ = make_inputs(cfg)
    p = O.to_f64(params)
    tab = O.modulation_table(params, cfg)
    assert tab.shape == (cfg.num_steps, 5, 3, cfg.width)
    # step 0 is t = 1, the last step is t = 1/N
    for k, t in ((0, 1.0), (cfg.num_steps - 1, 1.0 / cfg.num_steps)):
        c = O.time_conditioning(p, t)
        m = c @ p["layers.1.mlp_norm.mod.w"] + p["layers.1.mlp_norm.mod.b"]
        np.testing.assert_allclose(tab[k, 3].reshape(-1), m, atol=1e-15)


def test_gemm_input_amax_records_the_gemm_inputs():
    """The calibration recorder: at N = 1, L = 1 every GEMM input can be
    rebuilt from the oracle's public pieces; its largest |value| must be
    what the recorder keeps."""
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32"].replace(num_layers=1, num_steps=1)
    params, pk, pv, noise, state = make_inputs(cfg)
    p = O.to_f64(params)
    rec = O.gemm_input_amax(params, noise, state, pk, pv, cfg)
    c = O.time_conditioning(p, 1.0)
    h = noise.astype(np.float64) @ p["in_proj.w"] + p["in_proj.b"]
    sc, sh, g = O.modulation(c, p["layers.0.attn_norm.mod.w"], p["layers.0.attn_norm.mod.b"])
    xn = O.ada_rms_norm(h, sc, sh, cfg.rms_eps)
    assert rec[0, 0] == np.max(np.abs(xn))
    B, T, W = h.shape
    d, Hq = cfg.head_dim, cfg.num_q_heads
    q = O.rope((xn @ p["layers.0.q.w"]).reshape(B, T, Hq, d).transpose(0, 2, 1, 3), np.arange(64, 64 + T), 10000.0)
    k = O.rope((xn @ p["layers.0.k.w"]).reshape(B, T, 1, d).transpose(0, 2, 1, 3), np.arange(64, 64 + T), 10000.0)
    v = (xn @ p["layers.0.v.w"]).reshape(B, T, 1, d).transpose(0, 2, 1, 3)
    K = np.concatenate([pk[0].astype(np.float64).transpose(0, 2, 1, 3), k], axis=2)
    V = np.concatenate([pv[0].astype(np.float64).transpose(0, 2, 1, 3), v], axis=2)
    o = O.gqa_attention(q, K, V).transpose(0, 2, 1, 3).reshape(B, T, Hq * d)
    np.testing.assert_allclose(rec[0, 1], np.max(np.abs(o)), rtol=1e-12)
    h2 = h + g * (o @ p["layers.0.o.w"])
    sc, sh, g = O.modulation(c, p["layers.0.mlp_norm.mod.w"], p["layers.0.mlp_norm.mod.b"])
    xn2 = O.ada_rms_norm(h2, sc, sh, cfg.rms_eps)
    np.testing.assert_allclose(rec[0, 2], np.max(np.abs(xn2)), rtol=1e-12)
    a = O.gelu_tanh(xn2 @ p["layers.0.gate.w"]) * (xn2 @ p["layers.0.up.w"])
    np.testing.assert_allclose(rec[0, 3], np.max(np.abs(a)), rtol=1e-12)


def test_calibration_inputs_are_a_separate_draw():
    from synth import CONFIGS, make_calibration_inputs, make_inputs
    cfg = CONFIGS["tiny_fp32"]
    _, pk, pv, noise, state = make_inputs(cfg)
    cpk, cpv, cnoise, cstate = make_calibration_inputs(cfg)
    assert cpk.shape == pk.shape and cpv.shape == pv.shape and cnoise.shape == noise.shape
    assert not np.array_equal(cpk, pk) and not np.array_equal(cnoise, noise)
