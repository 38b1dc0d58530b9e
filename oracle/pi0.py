"""CPU float64 oracle of the pi0 variant of the action expert.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
package's smoke check and the CPU-baseline leg of the benchmark use it. It
shares no code with the HIP path.

The pages name pi0 beside pi0.5 among the models both runtimes serve (the
PhyAI summary's model list, the FlashRT forum post's supported VLAs) but
print neither's expert. The pi0.5 reading lives in `denoise.py`; pi0 differs
in how time and the robot state enter. The plainest reading, used by both
sides:

* Tokens: per sample one state token followed by the H action tokens
  (T = H + 1); the state token's input is state W_s + b_s.
* Action tokens: a = x W_in + b_in, e = sincos(t) of width W (R2's
  embedding), u = SiLU([a ; e] W_mi + b_mi), input = u W_mo + b_mo: the time
  enters through this MLP only, never through the norms.
* Blocks: pre-norm with plain RMSNorm and a (1 + w) gain, ungated residuals,
  the same attention (RoPE at positions P..P+H, GQA, prefix used as given)
  and GeGLU MLP as pi0.5.
* Attention mask: the state token sees the prefix and itself; every action
  token sees the prefix, the state token and all action tokens.
* Output: final (1 + w) RMSNorm of the action tokens, then W_out, b_out; the
  Euler loop is R1's.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .denoise import gelu_tanh, rms_normalize, rope, silu, sincos_embedding, to_f64

__all__ = ["gain_norm", "action_time_input", "suffix_attention", "pi0_layer", "velocity_pi0", "denoise_pi0"]


def gain_norm(h: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    return rms_normalize(h, eps) * (1.0 + w)


def action_time_input(p, x: np.ndarray, t: float) -> np.ndarray:
    """Action-token inputs [B, H, W]: SiLU([x W_in + b_in ; sincos(t)] W_mi + b_mi) W_mo + b_mo."""
    a = x @ p["in_proj.w"] + p["in_proj.b"]
    W = a.shape[-1]
    e = np.broadcast_to(sincos_embedding(t, W), a.shape)
    u = silu(np.concatenate([a, e], axis=-1) @ p["time_mlp_in.w"] + p["time_mlp_in.b"])
    return u @ p["time_mlp_out.w"] + p["time_mlp_out.b"]


def suffix_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, P: int) -> np.ndarray:
    """q [B, Hq, T, d]; k / v [B, Hkv, P + T, d] (prefix keys first). Token 0
    of the suffix (the state token) sees keys 0..P only; the others see all."""
    B, Hq, T, d = q.shape
    group = Hq // k.shape[1]
    kk = np.repeat(k, group, axis=1)
    vv = np.repeat(v, group, axis=1)
    s = np.einsum("bhtd,bhsd->bhts", q, kk) / math.sqrt(d)
    s[:, :, 0, P + 1:] = -np.inf
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("bhts,bhsd->bhtd", w, vv)


def pi0_layer(p, l: int, h: np.ndarray, pk: np.ndarray, pv: np.ndarray, cfg) -> np.ndarray:
    """One block over the suffix h [B, T, W]; pk / pv [B, P, Hkv, d]."""
    B, T, W = h.shape
    Hq, Hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    P = pk.shape[1]
    pre = f"layers.{l}."
    xn = gain_norm(h, p[pre + "attn_norm.w"], cfg.rms_eps)
    pos = np.arange(P, P + T)
    q = rope((xn @ p[pre + "q.w"]).reshape(B, T, Hq, d).transpose(0, 2, 1, 3), pos, cfg.rope_base)
    k = rope((xn @ p[pre + "k.w"]).reshape(B, T, Hkv, d).transpose(0, 2, 1, 3), pos, cfg.rope_base)
    v = (xn @ p[pre + "v.w"]).reshape(B, T, Hkv, d).transpose(0, 2, 1, 3)
    K = np.concatenate([pk.transpose(0, 2, 1, 3), k], axis=2)
    V = np.concatenate([pv.transpose(0, 2, 1, 3), v], axis=2)
    o = suffix_attention(q, K, V, P).transpose(0, 2, 1, 3).reshape(B, T, Hq * d)
    h = h + o @ p[pre + "o.w"]
    xn = gain_norm(h, p[pre + "mlp_norm.w"], cfg.rms_eps)
    return h + (gelu_tanh(xn @ p[pre + "gate.w"]) * (xn @ p[pre + "up.w"])) @ p[pre + "down.w"]


def velocity_pi0(p, x: np.ndarray, s: np.ndarray, t: float, prefix_k: np.ndarray, prefix_v: np.ndarray,
                 cfg) -> np.ndarray:
    """v(x, t) [B, H, A]; s = state W_s + b_s [B, W]; prefix_k/v [L, B, P, Hkv, d]."""
    h = np.concatenate([s[:, None, :], action_time_input(p, x, t)], axis=1)
    for l in range(cfg.num_layers):
        h = pi0_layer(p, l, h, prefix_k[l], prefix_v[l], cfg)
    return gain_norm(h[:, 1:], p["final_norm.w"], cfg.rms_eps) @ p["out_proj.w"] + p["out_proj.b"]


def denoise_pi0(params, noise: np.ndarray, state: np.ndarray, prefix_k: np.ndarray, prefix_v: np.ndarray, cfg,
                num_steps: Optional[int] = None) -> np.ndarray:
    """Euler from t = 1 (x = noise) to t = 0 in N steps of dt = -1/N (R1)."""
    p = params if all(v.dtype == np.float64 for v in params.values()) else to_f64(params)
    N = cfg.num_steps if num_steps is None else num_steps
    x = np.asarray(noise, dtype=np.float64).copy()
    pk = np.asarray(prefix_k, dtype=np.float64)
    pv = np.asarray(prefix_v, dtype=np.float64)
    s = np.asarray(state, dtype=np.float64) @ p["state_proj.w"] + p["state_proj.b"]
    for k in range(N):
        x = x + (-1.0 / N) * velocity_pi0(p, x, s, (N - k) / N, pk, pv, cfg)
    return x
