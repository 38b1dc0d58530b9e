"""Pins of the oracle's quantisers: the OCP e4m3 bit layout, round-to-nearest-
even with saturation, torch's CPU float8 cast on in-range values, and the
int4 group quantiser's grid and error bound."""
import numpy as np
import pytest
import torch

from oracle import quant as Q


def test_e4m3_decode_spec_values():
    dec = Q.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert dec[0x7E] == 448.0 and dec[0xFE] == -448.0
    assert dec[0x08] == 2.0 ** -6            # smallest normal
    assert dec[0x01] == 2.0 ** -9            # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert dec[0x38] == 1.0                  # exponent field 7 = bias
    assert dec[0x3C] == 1.5
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert np.sum(np.isnan(dec)) == 2
    assert dec[0x00] == 0.0 and dec[0x80] == 0.0
    finite = dec[~np.isnan(dec)]
    assert np.all(np.isfinite(finite))
    pos = Q.e4m3_all_values()
    assert np.all(np.diff(pos) > 0)


def test_e4m3_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(Q.e4m3_encode(Q.e4m3_decode(codes)), codes)


def test_e4m3_ties_to_even_and_saturation():
    pos = Q.e4m3_all_values()
    mids = (pos[:-1] + pos[1:]) / 2
    enc = Q.e4m3_encode(mids).astype(int)
    lo = np.arange(len(mids))
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, expect)
    assert Q.e4m3_encode(np.array([1e9]))[0] == 0x7E
    assert Q.e4m3_encode(np.array([-500.0]))[0] == 0xFE
    assert Q.e4m3_encode(np.array([np.nan]))[0] == 0x7F
    assert Q.e4m3_encode(np.array([2.0 ** -11]))[0] == 0x00   # below half the smallest subnormal -> 0
    assert Q.e4m3_encode(np.array([3 * 2.0 ** -11]))[0] == 0x01


def test_e4m3_vs_torch_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0, 120.0)]).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ours = Q.e4m3_decode(Q.e4m3_encode(x))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_tensor_quantiser():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 48)) * 0.02).astype(np.float32)
    codes, scale, deq = Q.quantise_fp8_tensor(w)
    assert scale == np.float32(np.max(np.abs(w)) / np.float32(448.0))
    assert np.max(np.abs(Q.e4m3_decode(codes))) == 448.0       # the amax element maps to the top code
    rel = np.abs(deq - w) / np.maximum(np.abs(w), 2.0 ** -6 * scale)
    assert np.max(rel) <= 2.0 ** -4 + 1e-12                     # half an ulp of a 3-bit mantissa
    z, s0, d0 = Q.quantise_fp8_tensor(np.zeros((4, 4), np.float32))
    assert s0 == 1.0 and np.all(d0 == 0)


def test_w4_quantiser():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((256, 40)) * 0.02).astype(np.float32)
    q, s, deq = Q.quantise_w4(w, 128)
    assert q.dtype == np.int8 and q.min() >= -8 and q.max() <= 7
    assert s.shape == (2, 40) and s.dtype == np.float16
    s32 = np.repeat(s.astype(np.float64), 128, axis=0)
    # rounding error at most half a step; amax/7 rounded to fp16 keeps the clip error below that too
    assert np.all(np.abs(deq - w) <= s32 / 2 + 1e-12)
    # values already on the grid round-trip exactly
    grid = (q.astype(np.float32) * np.repeat(s.astype(np.float32), 128, axis=0)).astype(np.float32)
    q2, s2, deq2 = Q.quantise_w4(grid, 128)
    assert np.array_equal(deq2, grid.astype(np.float64))
    # each group's largest magnitude maps to +-7 (or -8 is never needed for symmetric amax)
    assert np.all(np.max(np.abs(q.reshape(2, 128, 40)), axis=1) == 7)
    # an all-zero group gets scale 1 and codes 0
    w[:128, 3] = 0
    q3, s3, d3 = Q.quantise_w4(w, 128)
    assert s3[0, 3] == 1.0 and np.all(q3[:128, 3] == 0)


def test_dequantised_expert_fp8_shares_fused_scales():
    """FP8 quantises [q | k | v] and [gate | up] as single tensors: every
    fused part sits on the e4m3 grid of the one scale amax(fused) / 448."""
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32"].replace(weight_precision="fp8", num_layers=1)
    params, *_ = make_inputs(cfg)
    deq, scales = Q.dequantised_expert(params, cfg)
    grid = np.concatenate([-Q.e4m3_all_values()[::-1], Q.e4m3_all_values()])
    for gi, names in enumerate([["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]):
        mats = [params[f"layers.0.{n}.w"].astype(np.float32) for n in names]
        amax = max(float(np.max(np.abs(m))) for m in mats)
        assert scales[0, gi] == np.float32(np.float32(amax) / np.float32(448.0))
        for n in names:
            codes_val = deq[f"layers.0.{n}.w"] / np.float64(scales[0, gi])
            assert np.all(np.isin(codes_val, grid)), n
            # nearest-grid error bound: half a step of the local spacing (<= 1/16 relative above 2^-6),
            # plus the float32 rounding of the quotient w / scale that is encoded
            w = params[f"layers.0.{n}.w"].astype(np.float64)
            err = np.abs(deq[f"layers.0.{n}.w"] - w) / np.float64(scales[0, gi])
            assert np.all(err <= np.maximum(np.abs(w) / np.float64(scales[0, gi]) / 16.0, 2.0 ** -10) * (1 + 1e-6)), n
    # the tensor with the largest amax uses its full range
    assert np.max(np.abs(deq["layers.0.o.w"])) == np.float64(448.0) * np.float64(scales[0, 1])


def test_dequantised_expert_w4_is_per_matrix():
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32"].replace(weight_precision="w4a16", num_layers=1)
    params, *_ = make_inputs(cfg)
    deq, scales = Q.dequantised_expert(params, cfg)
    assert scales is None
    for n in ("q", "k", "v", "o", "gate", "up", "down"):
        _, _, d1 = Q.quantise_w4(params[f"layers.0.{n}.w"], 128)
        assert np.array_equal(deq[f"layers.0.{n}.w"], d1), n
    assert deq["in_proj.w"] is params["in_proj.w"]


def test_w8_quantiser():
    """Per-column int8: the scale is exactly amax / 127 in float32, codes in
    [-127, 127] with every column's largest magnitude at +-127, error at most
    half a step, ties to even, grid values round-trip, zero columns get
    scale 1; cross-checked against torch's own float32 division and
    round-half-even."""
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((192, 24)) * 0.02).astype(np.float32)
    w[:, 5] = 0.0
    q, s, deq = Q.quantise_w8(w)
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    amax = np.max(np.abs(w), axis=0)
    for n in range(24):
        want = np.float32(1.0) if amax[n] == 0 else np.float32(amax[n] / np.float32(127.0))
        assert s[n] == want
    live = amax > 0
    assert np.all(np.max(np.abs(q[:, live].astype(np.int64)), axis=0) == 127)
    assert s[5] == 1.0 and np.all(q[:, 5] == 0)
    assert np.all(np.abs(deq - w.astype(np.float64)) <= s.astype(np.float64)[None, :] / 2 * (1 + 1e-6))
    tq = torch.clamp(torch.round(torch.from_numpy(w) / torch.from_numpy(s)[None, :]), -127, 127).to(torch.int8)
    assert np.array_equal(tq.numpy(), q)
    # exact half steps round to the even code
    s1 = np.float32(0.5)
    ww = np.array([[127 * 0.5], [0.75], [1.25], [-0.75], [0.25]], dtype=np.float32)   # quotients 127, 1.5, 2.5, -1.5, 0.5
    qq, ss, _ = Q.quantise_w8(ww)
    assert ss[0] == s1
    assert qq[:, 0].tolist() == [127, 2, 2, -2, 0]
    # values on the grid keep their codes (the rescale is exact up to float32 rounding of 127 s)
    grid = (q.astype(np.float32) * s[None, :]).astype(np.float32)
    q2, s2, d2 = Q.quantise_w8(grid)
    assert np.array_equal(q2, q)
    assert np.all(np.abs(s2 / s - 1.0) <= 2.0 ** -22)


def test_dequantised_expert_w8_is_per_column():
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32"].replace(weight_precision="w8a16", num_layers=1)
    params, *_ = make_inputs(cfg)
    deq, scales = Q.dequantised_expert(params, cfg)
    assert scales is None
    for n in ("q", "k", "v", "o", "gate", "up", "down"):
        _, _, d1 = Q.quantise_w8(params[f"layers.0.{n}.w"])
        assert np.array_equal(deq[f"layers.0.{n}.w"], d1), n
        # slicing columns quantises identically (per-column scales ignore fusion)
        m = params[f"layers.0.{n}.w"]
        _, _, d2 = Q.quantise_w8(m[:, : m.shape[1] // 2])
        assert np.array_equal(d2, d1[:, : m.shape[1] // 2])


def test_dequantised_expert_w4a8_is_the_int4_group_grid():
    """The W4A8 branch (int4 weights, e4m3 activations): every GEMM weight is
    an integer code in [-8, 7] times the fp16 scale of its (128-row group,
    column), the scale being the group's largest magnitude over 7 rounded to
    fp16; each value lies within half a step of the bf16 master, each group's
    largest magnitude takes code +-7, and the weights outside the GEMMs pass
    through untouched. Checked from the definition, group by group, without
    the oracle's quantiser."""
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32"].replace(weight_precision="w4a8", num_layers=2)
    params, *_ = make_inputs(cfg)
    deq, scales = Q.dequantised_expert(params, cfg)
    assert scales is None
    G = cfg.w4_group
    for l in range(cfg.num_layers):
        for n in ("q", "k", "v", "o", "gate", "up", "down"):
            w = params[f"layers.{l}.{n}.w"].astype(np.float64)
            d = np.asarray(deq[f"layers.{l}.{n}.w"], dtype=np.float64)
            K, N = w.shape
            assert d.shape == (K, N)
            for g0 in range(0, K, G):
                for c in range(N):
                    col = w[g0:g0 + G, c]
                    amax = float(np.max(np.abs(col)))
                    s = float(np.float16(np.float32(amax) / np.float32(7.0))) if amax > 0 else 1.0
                    codes = d[g0:g0 + G, c] / s
                    assert np.all(codes == np.round(codes)), (l, n, g0, c)
                    assert codes.min() >= -8 and codes.max() <= 7
                    assert np.all(np.abs(d[g0:g0 + G, c] - col) <= s / 2 * (1 + 1e-6) + 1e-300)
                    if amax > 0:
                        assert np.max(np.abs(codes)) == 7.0
    for name in ("in_proj.w", "out_proj.w", "time_mlp_in.w"):
        if name in params:
            assert deq[name] is params[name]
