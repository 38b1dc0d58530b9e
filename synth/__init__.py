"""Seeded synthetic inputs for the flow-matching action expert.

This module is shared by the CPU oracle tests and the GPU path. It holds the
workload shapes and the random draws only; none of the method's arithmetic
lives here. Every array is returned as numpy float32. For 16-bit configs the
draws are rounded (round-to-nearest-even) onto the bfloat16 grid so that both
sides read exactly the same values; that rounding is a storage conversion of
the inputs, not part of the method.

Draw order (one ``numpy.random.Generator(PCG64(seed))`` per workload):
time MLP -> in/state projections -> layers 0..L-1 (attn mod, q, k, v, o,
mlp mod, gate, up, down) -> final mod -> out projection -> prefix K ->
prefix V -> noise -> state. Weights and biases are N(0, 0.02^2); prefix K/V,
noise and state are N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

__all__ = ["ExpertConfig", "CONFIGS", "param_specs", "make_params", "make_inputs",
           "make_calibration_inputs", "round_to_bf16", "workload", "PrefixConfig", "PREFIX_CONFIGS",
           "prefix_param_specs", "make_prefix_inputs"]


@dataclasses.dataclass(frozen=True)
class ExpertConfig:
    name: str
    num_layers: int
    width: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    mlp_dim: int
    action_horizon: int
    action_dim: int
    state_dim: int
    time_emb_dim: int
    prefix_len: int
    batch: int
    num_steps: int = 10
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    weight_precision: str = "fp32"     # fp32 | bf16 | fp8 | w4a16 | w8a16 | w4a8
    w4_group: int = 128
    seed: int = 0
    weight_std: float = 0.02
    variant: str = "pi05"              # pi05: adaptive norms; pi0: state token + action-time MLP

    @property
    def act_dtype(self) -> str:
        """Storage type of GEMM activations on the GPU path."""
        return "f32" if self.weight_precision == "fp32" else "bf16"

    @property
    def master_dtype(self) -> str:
        """Storage type of the master weights handed to the library."""
        return "f32" if self.weight_precision == "fp32" else "bf16"

    def replace(self, **kw) -> "ExpertConfig":
        return dataclasses.replace(self, **kw)


def _pi05(name: str, **kw) -> ExpertConfig:
    base = dict(name=name, num_layers=18, width=1024, num_q_heads=8, num_kv_heads=1,
                head_dim=256, mlp_dim=4096, action_horizon=50, action_dim=32, state_dim=32,
                time_emb_dim=1024, prefix_len=560, batch=1, weight_precision="bf16")
    base.update(kw)
    return ExpertConfig(**base)


# The five workloads: a tiny fp32 correctness expert and a pi0.5-shaped expert
# at batch 1 (bf16, FP8 with a 3-view prefix, W4A16) and batch 32.
CONFIGS: Dict[str, ExpertConfig] = {
    "tiny_fp32": ExpertConfig(name="tiny_fp32", num_layers=2, width=256, num_q_heads=4,
                              num_kv_heads=1, head_dim=64, mlp_dim=1024, action_horizon=8,
                              action_dim=8, state_dim=0, time_emb_dim=256, prefix_len=64,
                              batch=1, weight_precision="fp32", seed=0),
    "pi05_bf16_b1": _pi05("pi05_bf16_b1", seed=1),
    "pi05_fp8_p816": _pi05("pi05_fp8_p816", prefix_len=816, weight_precision="fp8", seed=2),
    "pi05_w4a16": _pi05("pi05_w4a16", weight_precision="w4a16", seed=3),
    "pi05_bf16_b32": _pi05("pi05_bf16_b32", batch=32, seed=4),
    "pi05_w8a16": _pi05("pi05_w8a16", weight_precision="w8a16", seed=5),
    "pi05_w4a8": _pi05("pi05_w4a8", weight_precision="w4a8", seed=6),
    # pi0: a state token before the action tokens, the time folded into the
    # action tokens by an MLP, plain norms
    "pi0_tiny_fp32": ExpertConfig(name="pi0_tiny_fp32", num_layers=2, width=256, num_q_heads=4, num_kv_heads=1,
                                  head_dim=64, mlp_dim=1024, action_horizon=8, action_dim=8, state_dim=8,
                                  time_emb_dim=256, prefix_len=64, batch=1, weight_precision="fp32", seed=20,
                                  variant="pi0"),
    "pi0_bf16_b1": _pi05("pi0_bf16_b1", seed=21, variant="pi0"),
}


def workload(name: str) -> ExpertConfig:
    return CONFIGS[name]


def _pi0_specs(cfg: ExpertConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    W, A, S, F = cfg.width, cfg.action_dim, cfg.state_dim, cfg.mlp_dim
    qd, kd = cfg.num_q_heads * cfg.head_dim, cfg.num_kv_heads * cfg.head_dim
    specs: List[Tuple[str, Tuple[int, ...]]] = [
        ("time_mlp_in.w", (2 * W, W)), ("time_mlp_in.b", (W,)),
        ("time_mlp_out.w", (W, W)), ("time_mlp_out.b", (W,)),
        ("in_proj.w", (A, W)), ("in_proj.b", (W,)),
        ("state_proj.w", (S, W)), ("state_proj.b", (W,)),
    ]
    for l in range(cfg.num_layers):
        p = f"layers.{l}."
        specs += [(p + "attn_norm.w", (W,)), (p + "q.w", (W, qd)), (p + "k.w", (W, kd)), (p + "v.w", (W, kd)),
                  (p + "o.w", (qd, W)), (p + "mlp_norm.w", (W,)), (p + "gate.w", (W, F)), (p + "up.w", (W, F)),
                  (p + "down.w", (F, W))]
    specs += [("final_norm.w", (W,)), ("out_proj.w", (W, A)), ("out_proj.b", (A,))]
    return specs


def param_specs(cfg: ExpertConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """Canonical parameter names and shapes, in draw order. All matrices are
    stored [in][out] (y = x @ W). The pi0 variant has an action-time MLP
    ([action ; time] 2W -> W -> W), a state projection and plain (1 + w)
    norm weights instead of the modulation layers."""
    if cfg.variant == "pi0":
        return _pi0_specs(cfg)
    W, E, A, S = cfg.width, cfg.time_emb_dim, cfg.action_dim, cfg.state_dim
    qd = cfg.num_q_heads * cfg.head_dim
    kd = cfg.num_kv_heads * cfg.head_dim
    F = cfg.mlp_dim
    specs: List[Tuple[str, Tuple[int, ...]]] = [
        ("time_mlp_in.w", (E, W)), ("time_mlp_in.b", (W,)),
        ("time_mlp_out.w", (W, W)), ("time_mlp_out.b", (W,)),
        ("in_proj.w", (A, W)), ("in_proj.b", (W,)),
    ]
    if S > 0:
        specs += [("state_proj.w", (S, W)), ("state_proj.b", (W,))]
    for l in range(cfg.num_layers):
        p = f"layers.{l}."
        specs += [
            (p + "attn_norm.mod.w", (W, 3 * W)), (p + "attn_norm.mod.b", (3 * W,)),
            (p + "q.w", (W, qd)), (p + "k.w", (W, kd)), (p + "v.w", (W, kd)), (p + "o.w", (qd, W)),
            (p + "mlp_norm.mod.w", (W, 3 * W)), (p + "mlp_norm.mod.b", (3 * W,)),
            (p + "gate.w", (W, F)), (p + "up.w", (W, F)), (p + "down.w", (F, W)),
        ]
    specs += [("final_norm.mod.w", (W, 3 * W)), ("final_norm.mod.b", (3 * W,)),
              ("out_proj.w", (W, A)), ("out_proj.b", (A,))]
    return specs


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32. NaN/Inf do not occur in these draws."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _draw(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_params(cfg: ExpertConfig, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    params: Dict[str, np.ndarray] = {}
    for name, shape in param_specs(cfg):
        a = _draw(rng, shape, cfg.weight_std)
        if cfg.master_dtype == "bf16":
            a = round_to_bf16(a)
        params[name] = a
    return params


def make_inputs(cfg: ExpertConfig, seed: int | None = None):
    """Return (params, prefix_k, prefix_v, noise, state) for a workload.

    prefix_k / prefix_v: [L][B][P][Hkv][d]; noise: [B][H][A]; state: [B][S]
    (a [B][0] array when the expert has no state input)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    params = make_params(cfg, rng)
    kv_shape = (cfg.num_layers, cfg.batch, cfg.prefix_len, cfg.num_kv_heads, cfg.head_dim)
    pk = rng.standard_normal(size=kv_shape, dtype=np.float32)
    pv = rng.standard_normal(size=kv_shape, dtype=np.float32)
    if cfg.act_dtype == "bf16":
        pk, pv = round_to_bf16(pk), round_to_bf16(pv)
    noise = rng.standard_normal(size=(cfg.batch, cfg.action_horizon, cfg.action_dim), dtype=np.float32)
    state = rng.standard_normal(size=(cfg.batch, cfg.state_dim), dtype=np.float32)
    return params, pk, pv, noise, state


def make_calibration_inputs(cfg: ExpertConfig):
    """The inputs of an FP8 calibration pass, drawn apart from the evaluation
    inputs: one ``PCG64(seed + 1000)`` generator, in the order prefix K,
    prefix V, noise, state (same shapes and distributions as make_inputs)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed + 1000))
    kv_shape = (cfg.num_layers, cfg.batch, cfg.prefix_len, cfg.num_kv_heads, cfg.head_dim)
    pk = rng.standard_normal(size=kv_shape, dtype=np.float32)
    pv = rng.standard_normal(size=kv_shape, dtype=np.float32)
    if cfg.act_dtype == "bf16":
        pk, pv = round_to_bf16(pk), round_to_bf16(pv)
    noise = rng.standard_normal(size=(cfg.batch, cfg.action_horizon, cfg.action_dim), dtype=np.float32)
    state = rng.standard_normal(size=(cfg.batch, cfg.state_dim), dtype=np.float32)
    return pk, pv, noise, state


def make_noise_state(cfg: ExpertConfig, seed: int):
    """A fresh (noise, state) draw, e.g. for a calibration pass that must not
    see the evaluation inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    noise = rng.standard_normal(size=(cfg.batch, cfg.action_horizon, cfg.action_dim), dtype=np.float32)
    state = rng.standard_normal(size=(cfg.batch, cfg.state_dim), dtype=np.float32)
    return noise, state


# ---------------------------------------------------------------------------
# The prefix producer: a Gemma-2B-shaped decoder run once over the
# vision + language prefix, whose per-layer keys and values are the prefix
# K/V the action expert attends to.
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class PrefixConfig:
    name: str
    num_layers: int
    width: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    mlp_dim: int
    prefix_len: int
    batch: int
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    seed: int = 0
    weight_std: float = 0.02

    def replace(self, **kw) -> "PrefixConfig":
        return dataclasses.replace(self, **kw)


PREFIX_CONFIGS: Dict[str, PrefixConfig] = {
    # small correctness case: a prefix that is not a multiple of any tile
    "prefix_tiny": PrefixConfig(name="prefix_tiny", num_layers=2, width=256, num_q_heads=4, num_kv_heads=1,
                                head_dim=64, mlp_dim=512, prefix_len=100, batch=1, seed=10),
    # Gemma-2B shape (18 layers, width 2048, 8 query heads sharing one KV head of
    # dim 256, GeGLU 16384) over 2 views x 256 image tokens + 48 text tokens
    "prefix_gemma2b_p560": PrefixConfig(name="prefix_gemma2b_p560", num_layers=18, width=2048, num_q_heads=8,
                                        num_kv_heads=1, head_dim=256, mlp_dim=16384, prefix_len=560, batch=1,
                                        seed=11),
}


def prefix_param_specs(cfg: PrefixConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """Names and shapes of the prefix decoder's weights, in draw order
    (matrices [in][out]; norm weights are the w of a (1 + w) gain)."""
    W, F = cfg.width, cfg.mlp_dim
    qd, kd = cfg.num_q_heads * cfg.head_dim, cfg.num_kv_heads * cfg.head_dim
    specs: List[Tuple[str, Tuple[int, ...]]] = []
    for l in range(cfg.num_layers):
        p = f"layers.{l}."
        specs += [(p + "attn_norm.w", (W,)), (p + "q.w", (W, qd)), (p + "k.w", (W, kd)), (p + "v.w", (W, kd)),
                  (p + "o.w", (qd, W)), (p + "mlp_norm.w", (W,)), (p + "gate.w", (W, F)), (p + "up.w", (W, F)),
                  (p + "down.w", (F, W))]
    return specs


def make_prefix_inputs(cfg: PrefixConfig, seed: int | None = None):
    """Return (params, embeds): bf16-grid weights N(0, std^2) in draw order,
    then the prefix token embeddings [B][P][W] N(0, 1) on the bf16 grid (they
    stand in for the image-encoder outputs and text-token embeddings)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    params = {n: round_to_bf16(_draw(rng, s, cfg.weight_std)) for n, s in prefix_param_specs(cfg)}
    embeds = round_to_bf16(rng.standard_normal(size=(cfg.batch, cfg.prefix_len, cfg.width), dtype=np.float32))
    return params, embeds
