"""CPU float64 oracle of the flow-matching action expert's denoise loop.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the tests, the package's smoke check and the CPU-baseline
leg of the benchmark do. It shares no code with the HIP path.

What it computes. The pages (the PhyAI summary, "Real-Time Physical AI at the
Edge, Scalable Rollouts in the Cloud", its optimisation paragraph and its
profiling paragraph) describe pi0.5's action expert as a ten-step Euler
iteration of a flow-matching policy whose small transformer runs over the
action-chunk tokens and attends to a cached vision+language prefix. They do
not print the expert's equations, so every formula below is the plainest
reading of that description, stated where it is used:

* Euler: t_k = (N-k)/N for k = 0..N-1, x <- x + dt * v(x, t_k), dt = -1/N,
  so a constant field v carries x(1) to x(1) - v at t = 0.
* Time conditioning: sinusoidal embedding of t, then a two-layer MLP
  (E -> W -> W) with SiLU after each layer.
* adaRMSNorm: y = x / sqrt(mean(x^2) + eps) * (1 + scale) + shift, with
  (scale, shift, gate) = c @ W_mod + b_mod per norm; every one of the 2L+1
  norms is adaptive; residual branches are gated: h <- h + gate * branch.
* Attention: grouped-query, every action token attends to all P prefix keys
  and all H chunk keys (no mask), softmax(q k^T / sqrt(d)) v; rotary encoding
  (half-split pairs (j, j + d/2), inv_freq_j = base^(-2j/d)) on q and the
  chunk's k at absolute positions P..P+H-1; prefix keys are used as given.
* MLP: GeGLU with the tanh form of GELU.
* No biases on q/k/v/o/gate/up/down; biases on in/out/state projections,
  the time MLP and the modulation layers.
* State: s = state @ W_s + b_s is added to every action token's input.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

__all__ = ["sincos_embedding", "silu", "time_conditioning", "modulation", "rms_normalize",
           "ada_rms_norm", "rope", "gqa_attention", "gelu_tanh", "expert_layer",
           "velocity", "denoise", "gemm_input_amax", "modulation_table", "to_f64"]


def to_f64(params: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Inputs are converted to float64 exactly as stored."""
    return {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}


def sincos_embedding(t: float, dim: int, min_period: float = 4e-3, max_period: float = 4.0) -> np.ndarray:
    """Sinusoidal embedding of a scalar time t in [0, 1]: dim/2 geometrically
    spaced periods between min_period and max_period; e = [sin(2 pi t / p) || cos(2 pi t / p)]."""
    half = dim // 2
    frac = np.arange(half, dtype=np.float64) / (half - 1)
    period = min_period * (max_period / min_period) ** frac
    arg = 2.0 * math.pi * float(t) / period
    return np.concatenate([np.sin(arg), np.cos(arg)])


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def time_conditioning(p: Dict[str, np.ndarray], t: float) -> np.ndarray:
    """c = SiLU(SiLU(e W1 + b1) W2 + b2), e = sincos(t). The trailing SiLU is the
    activation that precedes every modulation layer."""
    e = sincos_embedding(t, p["time_mlp_in.w"].shape[0])
    h = silu(e @ p["time_mlp_in.w"] + p["time_mlp_in.b"])
    return silu(h @ p["time_mlp_out.w"] + p["time_mlp_out.b"])


def modulation(c: np.ndarray, w: np.ndarray, b: np.ndarray):
    """(scale, shift, gate) = split3(c W_mod + b_mod), column order [scale | shift | gate]."""
    m = c @ w + b
    W = m.shape[-1] // 3
    return m[..., :W], m[..., W:2 * W], m[..., 2 * W:]


def rms_normalize(h: np.ndarray, eps: float) -> np.ndarray:
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def ada_rms_norm(h: np.ndarray, scale: np.ndarray, shift: np.ndarray, eps: float) -> np.ndarray:
    return rms_normalize(h, eps) * (1.0 + scale) + shift


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotary encoding over the last axis (size d) of x[..., T, d] at integer
    positions[T]; pairs are (j, j + d/2)."""
    d = x.shape[-1]
    half = d // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q [B, Hq, T, d], k/v [B, Hkv, Tk, d] -> [B, Hq, T, d].
    Query head j reads KV head j // (Hq / Hkv); no mask; max-subtracted softmax."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    kk = np.repeat(k, group, axis=1)
    vv = np.repeat(v, group, axis=1)
    s = np.einsum("bhtd,bhsd->bhts", q, kk) / math.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("bhts,bhsd->bhtd", p, vv)


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def _note(record, l: int, i: int, x: np.ndarray) -> None:
    """Keep the largest |x| of GEMM input i of layer l (0 qkv, 1 o, 2 gate/up, 3 down)."""
    if record is not None and x.size:
        record[l, i] = max(record[l, i], float(np.max(np.abs(x))))


def expert_layer(p, l: int, h: np.ndarray, c: np.ndarray, pk: np.ndarray, pv: np.ndarray, cfg,
                 record: Optional[np.ndarray] = None) -> np.ndarray:
    """One transformer block over h [B, H, W]; pk/pv [B, P, Hkv, d] for this layer.
    `record` ([L][4], optional) collects the largest |input| of each GEMM."""
    B, T, W = h.shape
    Hq, Hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    P = pk.shape[1]
    pre = f"layers.{l}."
    sc, sh, g = modulation(c, p[pre + "attn_norm.mod.w"], p[pre + "attn_norm.mod.b"])
    xn = ada_rms_norm(h, sc, sh, cfg.rms_eps)
    _note(record, l, 0, xn)
    q = (xn @ p[pre + "q.w"]).reshape(B, T, Hq, d).transpose(0, 2, 1, 3)
    k = (xn @ p[pre + "k.w"]).reshape(B, T, Hkv, d).transpose(0, 2, 1, 3)
    v = (xn @ p[pre + "v.w"]).reshape(B, T, Hkv, d).transpose(0, 2, 1, 3)
    pos = np.arange(P, P + T)
    q = rope(q, pos, cfg.rope_base)
    k = rope(k, pos, cfg.rope_base)
    K = np.concatenate([pk.transpose(0, 2, 1, 3), k], axis=2)   # [B, Hkv, P+T, d]
    V = np.concatenate([pv.transpose(0, 2, 1, 3), v], axis=2)
    o = gqa_attention(q, K, V).transpose(0, 2, 1, 3).reshape(B, T, Hq * d)
    _note(record, l, 1, o)
    h = h + g * (o @ p[pre + "o.w"])
    sc, sh, g = modulation(c, p[pre + "mlp_norm.mod.w"], p[pre + "mlp_norm.mod.b"])
    xn = ada_rms_norm(h, sc, sh, cfg.rms_eps)
    _note(record, l, 2, xn)
    a = gelu_tanh(xn @ p[pre + "gate.w"]) * (xn @ p[pre + "up.w"])
    _note(record, l, 3, a)
    return h + g * (a @ p[pre + "down.w"])


def velocity(p, x: np.ndarray, s: Optional[np.ndarray], t: float, prefix_k: np.ndarray,
             prefix_v: np.ndarray, cfg, record: Optional[np.ndarray] = None) -> np.ndarray:
    """Velocity field v(x, t) [B, H, A]; prefix_k/v [L, B, P, Hkv, d]."""
    c = time_conditioning(p, t)
    h = x @ p["in_proj.w"] + p["in_proj.b"]
    if s is not None:
        h = h + s[:, None, :]
    for l in range(cfg.num_layers):
        h = expert_layer(p, l, h, c, prefix_k[l], prefix_v[l], cfg, record)
    sc, sh, _ = modulation(c, p["final_norm.mod.w"], p["final_norm.mod.b"])
    return ada_rms_norm(h, sc, sh, cfg.rms_eps) @ p["out_proj.w"] + p["out_proj.b"]


def denoise(params, noise: np.ndarray, state: np.ndarray, prefix_k: np.ndarray,
            prefix_v: np.ndarray, cfg, num_steps: Optional[int] = None,
            record: Optional[np.ndarray] = None) -> np.ndarray:
    """Explicit Euler from t = 1 (x = noise) to t = 0 in N equal steps of dt = -1/N.
    Returns the action chunk [B, H, A] in float64. `record` ([L][4], optional)
    collects the largest |input| of every GEMM over all steps."""
    p = params if all(v.dtype == np.float64 for v in params.values()) else to_f64(params)
    N = cfg.num_steps if num_steps is None else num_steps
    x = np.asarray(noise, dtype=np.float64).copy()
    pk = np.asarray(prefix_k, dtype=np.float64)
    pv = np.asarray(prefix_v, dtype=np.float64)
    s = None
    if cfg.state_dim > 0:
        s = np.asarray(state, dtype=np.float64) @ p["state_proj.w"] + p["state_proj.b"]
    dt = -1.0 / N
    for k in range(N):
        t = (N - k) / N
        x = x + dt * velocity(p, x, s, t, pk, pv, cfg, record)
    return x


def gemm_input_amax(params, noise, state, prefix_k, prefix_v, cfg) -> np.ndarray:
    """[L][4] largest |input| of the qkv, o, gate/up and down GEMMs of every
    layer over one full denoise call: what an FP8 calibration pass measures
    (FlashRT walk-through, component 6: one measurement pass records the amax
    of every FP8 GEMM input)."""
    rec = np.zeros((cfg.num_layers, 4))
    denoise(params, noise, state, prefix_k, prefix_v, cfg, record=rec)
    return rec


def modulation_table(params, cfg, num_steps: Optional[int] = None) -> np.ndarray:
    """(scale, shift, gate) of every norm at every step: [N][2L+1][3][W], norm
    order attn_0, mlp_0, ..., attn_{L-1}, mlp_{L-1}, final."""
    p = params if all(v.dtype == np.float64 for v in params.values()) else to_f64(params)
    N = cfg.num_steps if num_steps is None else num_steps
    names = []
    for l in range(cfg.num_layers):
        names += [f"layers.{l}.attn_norm.mod", f"layers.{l}.mlp_norm.mod"]
    names.append("final_norm.mod")
    W = cfg.width
    out = np.zeros((N, len(names), 3, W))
    for k in range(N):
        c = time_conditioning(p, (N - k) / N)
        for i, n in enumerate(names):
            sc, sh, g = modulation(c, p[n + ".w"], p[n + ".b"])
            out[k, i] = np.stack([sc, sh, g])
    return out
