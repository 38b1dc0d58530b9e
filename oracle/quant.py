"""CPU oracle of the weight quantisers (FP8 e4m3 per-tensor, int4 group-wise,
int8 per output channel).

TEST INFRASTRUCTURE ONLY: imported by the tests and never by the product path.

The PhyAI summary ("Real-Time Physical AI at the Edge, Scalable Rollouts in the
Cloud", optimisation paragraph) lists offline W4A16, W8A16, W8A8 and W4A8
quantisation; the
FlashRT walk-through (component 6, calibration) describes FP8 GEMMs whose
alpha is the product of an activation scale and a weight scale. The pages fix
no rounding rule or format details, so this module takes the plainest reading:

* FP8 is the OCP e4m3 ("fn") format: 1 sign, 4 exponent bits (bias 7),
  3 mantissa bits, no infinities, 0x7F/0xFF are NaN, largest finite 448.
  Encoding rounds to nearest with ties to the even code and saturates at 448.
  A tensor's scale is amax/448 in float32 (1 if amax is 0); the code of w is
  the encoding of the float32 quotient w / scale.
* int4 is symmetric, per output column and per group of 128 consecutive K
  rows: s = float16(amax / 7) (1 if that is 0), q = clip(rint(w / s), -8, 7)
  with the division in float32; the dequantised weight is q * s.
* W8A16 weights are symmetric int8 per output column over the whole K:
  s = float32(amax / 127) (1 if amax is 0), q = clip(rint(w / s), -127, 127)
  with the division in float32 (rint: ties to even); the dequantised weight
  is q * s and the activations stay bf16.
"""
from __future__ import annotations

import numpy as np

__all__ = ["e4m3_decode", "e4m3_encode", "e4m3_all_values", "quantise_fp8_tensor",
           "quantise_w4", "quantise_w8", "dequantised_expert", "E4M3_MAX"]

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 e4m3 codes to float64 from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m / 8.0 * 2.0 ** -6
    norm = (1.0 + m / 8.0) * 2.0 ** (e - 7.0)
    val = np.where(e == 0, sub, norm)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_all_values() -> np.ndarray:
    """The 127 non-negative finite values, in code order 0x00..0x7E (ascending)."""
    return e4m3_decode(np.arange(0x7F, dtype=np.uint8))


_POS = e4m3_all_values()


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value (ties to the even code), saturating to
    +-448. NaN encodes as 0x7F. Works for float32 or float64 input (the
    comparison is exact in float64)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(a == _POS[hi], hi, code)
    neg = (x < 0) & (code != 0)
    code = np.where(neg, code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quantise_fp8_tensor(w: np.ndarray):
    """Per-tensor FP8 quantisation. Returns (codes uint8, scale float32,
    dequantised float64 = decode(code) * scale)."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.float32(np.max(np.abs(w32))) if w32.size else np.float32(0)
    scale = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    q = (w32 / scale).astype(np.float32)
    codes = e4m3_encode(q)
    deq = e4m3_decode(codes) * np.float64(scale)
    return codes, scale, deq


def quantise_w4(w: np.ndarray, group: int = 128):
    """Symmetric int4 per (output column, K-group). w is [K][N].
    Returns (q int8 [K][N], scales float16 [K/group][N], dequantised float64)."""
    w32 = np.asarray(w, dtype=np.float32)
    K, N = w32.shape
    assert K % group == 0
    g = w32.reshape(K // group, group, N)
    amax = np.max(np.abs(g), axis=1)                                   # [G][N]
    s16 = (amax / np.float32(7.0)).astype(np.float32).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    s32 = s16.astype(np.float32)
    q = np.clip(np.rint((g / s32[:, None, :]).astype(np.float32)), -8, 7).astype(np.int8)
    deq = q.astype(np.float64) * s32[:, None, :].astype(np.float64)
    return q.reshape(K, N), s16, deq.reshape(K, N)


def quantise_w8(w: np.ndarray):
    """Symmetric int8 per output column. w is [K][N]. Returns (q int8 [K][N],
    scales float32 [N], dequantised float64 = q * s)."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=0)                                   # [N], exact
    s = (amax / np.float32(127.0)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = np.clip(np.rint((w32 / s[None, :]).astype(np.float32)), -127, 127).astype(np.int8)
    deq = q.astype(np.float64) * s[None, :].astype(np.float64)
    return q, s, deq


def dequantised_expert(params, cfg):
    """The expert's parameters with every per-layer GEMM weight replaced by
    the float64 value its quantised form stands for (what the oracle is fed
    for the quantised experts). FP8 quantises each fused GEMM tensor as a
    whole, [q | k | v] and [gate | up] along the output columns, so the
    fused parts share one scale; int4 scales are per column, so fusion does
    not matter there (nor for the per-column int8 of W8A16). Also returns the
    FP8 weight scales [L][4] (qkv, o, gate/up, down), or None otherwise."""
    out = dict(params)
    L = cfg.num_layers
    if cfg.weight_precision == "fp8":
        scales = np.zeros((L, 4), dtype=np.float32)
        for l in range(L):
            pre = f"layers.{l}."
            groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
            for gi, names in enumerate(groups):
                mats = [np.asarray(params[pre + n + ".w"], dtype=np.float32) for n in names]
                _, scale, deq = quantise_fp8_tensor(np.concatenate(mats, axis=1))
                scales[l, gi] = scale
                c0 = 0
                for n, m in zip(names, mats):
                    out[pre + n + ".w"] = deq[:, c0:c0 + m.shape[1]]
                    c0 += m.shape[1]
        return out, scales
    if cfg.weight_precision in ("w4a16", "w8a16", "w4a8"):
        # W4A8 stores the weights of W4A16 (its e4m3 activations are the
        # kernels' rounding of the GEMM inputs, like FP8's)
        for l in range(L):
            pre = f"layers.{l}."
            for n in ("q", "k", "v", "o", "gate", "up", "down"):
                if cfg.weight_precision in ("w4a16", "w4a8"):
                    _, _, deq = quantise_w4(params[pre + n + ".w"], cfg.w4_group)
                else:
                    _, _, deq = quantise_w8(params[pre + n + ".w"])
                out[pre + n + ".w"] = deq
        return out, None
    raise ValueError(f"{cfg.weight_precision} weights are not quantised")
