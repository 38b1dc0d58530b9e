"""CPU float64 oracle of the prefix producer: the vision + language decoder
pass whose per-layer keys and values are the prefix K/V that the action
expert attends to.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
package's smoke check and the CPU-baseline leg of the benchmark use it. It
shares no code with the HIP path.

What it computes. The pages name the prefix only as the vision + language
part of pi0 / pi0.5 that the action expert reads through its cached keys and
values (the PhyAI summary's profiling paragraph: the expert's share of batch-1
latency is what remains after this pass), with a PaliGemma-family backbone.
They print none of its equations; the plainest reading, stated here and used
by both sides:

* a pre-norm decoder over the P prefix tokens of each sample; input = the
  token embeddings as given (no embedding lookup or scaling here);
* RMSNorm with a (1 + w) gain: y = x / sqrt(mean(x^2) + eps) * (1 + w);
* attention: grouped-query, every prefix token attends to every prefix token
  (one bidirectional block, no mask), softmax(q k^T / sqrt(d)) v; rotary
  encoding with half-split pairs (j, j + d/2) on q and k at positions
  0..P-1 (the action expert's chunk then sits at P..P+H-1);
* MLP: GeGLU with the tanh form of GELU; no biases anywhere;
* output: for every layer l, k_l = RoPE(norm(x_l) W_k) and v_l = norm(x_l) W_v,
  laid out [L][B][P][Hkv][d]. The last layer's attention output and MLP do
  not reach any output and are not computed.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .denoise import gelu_tanh, gqa_attention, rms_normalize, rope, to_f64

__all__ = ["gain_rms_norm", "prefix_layer_kv", "prefix_kv"]


def gain_rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * (1 + w)."""
    return rms_normalize(x, eps) * (1.0 + w)


def prefix_layer_kv(p: Dict[str, np.ndarray], l: int, x: np.ndarray, cfg, last: bool):
    """One decoder layer over x [B, P, W]. Returns (k, v, x_next) with k, v
    [B, P, Hkv, d] (k rotary-encoded); x_next is None when `last`."""
    B, P, W = x.shape
    Hq, Hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    pre = f"layers.{l}."
    xn = gain_rms_norm(x, p[pre + "attn_norm.w"], cfg.rms_eps)
    pos = np.arange(P)
    k = rope((xn @ p[pre + "k.w"]).reshape(B, P, Hkv, d).transpose(0, 2, 1, 3), pos, cfg.rope_base)
    v = (xn @ p[pre + "v.w"]).reshape(B, P, Hkv, d).transpose(0, 2, 1, 3)
    k_out, v_out = k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3)
    if last:
        return k_out, v_out, None
    q = rope((xn @ p[pre + "q.w"]).reshape(B, P, Hq, d).transpose(0, 2, 1, 3), pos, cfg.rope_base)
    o = gqa_attention(q, k, v).transpose(0, 2, 1, 3).reshape(B, P, Hq * d)
    x = x + o @ p[pre + "o.w"]
    xn = gain_rms_norm(x, p[pre + "mlp_norm.w"], cfg.rms_eps)
    a = gelu_tanh(xn @ p[pre + "gate.w"]) * (xn @ p[pre + "up.w"])
    return k_out, v_out, x + a @ p[pre + "down.w"]


def prefix_kv(params, embeds: np.ndarray, cfg):
    """(prefix_k, prefix_v), each [L][B][P][Hkv][d] float64, from the prefix
    token embeddings [B][P][W]."""
    p = params if all(v.dtype == np.float64 for v in params.values()) else to_f64(params)
    x = np.asarray(embeds, dtype=np.float64)
    L = cfg.num_layers
    B, P, _ = x.shape
    pk = np.zeros((L, B, P, cfg.num_kv_heads, cfg.head_dim))
    pv = np.zeros_like(pk)
    for l in range(L):
        pk[l], pv[l], x = prefix_layer_kv(p, l, x, cfg, last=(l == L - 1))
    return pk, pv
