"""GPU parity of the streaming batch-1 kernel (launch_mode "stream") through
the C ABI against the CPU fp64 oracle on the same seeded inputs.

Tolerances (bf16 weights and activations, fp32 accumulation and residual
stream): relative L2 of the actions <= 2e-3, relative L2 of the displacement
(actions - noise, the part the network contributes) <= 5e-3, and every
element of the displacement within 1e-2 of the largest reference
displacement. One bf16 rounding is 2^-9 = 2e-3 relative; the measured
errors at the pi0.5 batch-1 shape are 2.1e-4, 3.6e-4 and 4.6e-4, so the
bounds leave an order of magnitude for other seeds and shapes while a
dropped term or a wrong index (errors of order 1) fails all three.

The kernel is deterministic: the K-split partial sums are added in a fixed
order whichever workgroup arrives last, so repeated calls and calls with a
different loader depth (a timing-only setting) must agree bitwise."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import denoise as O
from synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

TOL_REL, TOL_DISP, TOL_ELEM = 2e-3, 5e-3, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_pi0_amd import vfm
    vfm.load_library()


def _gu():
    import gpu_util
    return gpu_util


def tiny_bf16(**kw):
    """The tiny expert with bf16 weights and a state input (stream-eligible shapes)."""
    return CONFIGS["tiny_fp32"].replace(name="tiny_bf16", weight_precision="bf16", state_dim=8, **kw)


_CACHE = {}


def case(cfg):
    key = repr(cfg)
    if key not in _CACHE:
        params, pk, pv, noise, state = make_inputs(cfg)
        ref = O.denoise(params, noise, state, pk, pv, cfg)
        _CACHE[key] = (params, pk, pv, noise, state, ref)
    return _CACHE[key]


def run_stream(cfg, params, pk, pv, noise, state, repeats=1, options=()):
    gu = _gu()
    ex = gu.build_expert(cfg, params, "stream")
    try:
        for k, v in options:
            ex.set_option(k, v)
        bufs = gu.bind_inputs(ex, cfg, pk, pv, noise, state)
        for _ in range(repeats):
            ex.denoise()
        ex.check()
        torch.cuda.synchronize()
        return bufs["actions"].cpu().numpy()
    finally:
        ex.close()


def check_parity(got, ref, noise, label):
    gu = _gu()
    err = gu.rel_l2(got, ref)
    disp = gu.rel_l2(got - noise, ref - noise)
    elem = float(np.max(np.abs((got - noise) - (ref - noise))) / np.max(np.abs(ref - noise)))
    print(f"{label}: rel_l2={err:.3e} displacement rel_l2={disp:.3e} max element {elem:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL_REL
    assert disp <= TOL_DISP
    assert elem <= TOL_ELEM


@pytest.mark.parametrize("which", ["tiny_bf16", "pi05_bf16_b1"])
def test_stream_matches_oracle(which):
    cfg = tiny_bf16() if which == "tiny_bf16" else CONFIGS["pi05_bf16_b1"]
    params, pk, pv, noise, state, ref = case(cfg)
    print(f"case {which} stream", flush=True)
    got = run_stream(cfg, params, pk, pv, noise, state, repeats=2)
    check_parity(got, ref, noise, which)


@pytest.mark.parametrize("prefix,horizon", [(37, 8), (130, 13), (5, 1), (64, 64), (250, 33)])
def test_stream_ragged_shapes(prefix, horizon):
    """Prefix lengths off the 32-key split, horizons off the 16-row MFMA tile
    (the last attention split, the padded token rows and the masked merge)."""
    cfg = tiny_bf16(prefix_len=prefix, action_horizon=horizon)
    params, pk, pv, noise, state, ref = case(cfg)
    print(f"case tiny_bf16 P={prefix} H={horizon}", flush=True)
    got = run_stream(cfg, params, pk, pv, noise, state)
    check_parity(got, ref, noise, f"P={prefix} H={horizon}")


def test_stream_longest_prefix():
    """pi0.5 shapes at the longest prefix of the configurations (816 tokens:
    28 key splits per head, the merge's widest pass)."""
    cfg = CONFIGS["pi05_bf16_b1"].replace(prefix_len=816)
    params, pk, pv, noise, state, ref = case(cfg)
    print("case pi05 bf16 P=816 stream", flush=True)
    got = run_stream(cfg, params, pk, pv, noise, state)
    check_parity(got, ref, noise, "pi05 P=816")


def test_stream_is_deterministic():
    cfg = CONFIGS["pi05_bf16_b1"]
    params, pk, pv, noise, state, _ = case(cfg)
    gu = _gu()
    ex = gu.build_expert(cfg, params, "stream")
    try:
        bufs = gu.bind_inputs(ex, cfg, pk, pv, noise, state)
        outs = []
        for cap in ("56", "56", "8", "32"):
            ex.set_option("stream_dma_cap", cap)
            ex.denoise()
            ex.check()
            torch.cuda.synchronize()
            outs.append(bufs["actions"].cpu().numpy())
        for o in outs[1:]:
            assert np.array_equal(o, outs[0])
    finally:
        ex.close()


def test_stream_agrees_with_persistent():
    cfg = CONFIGS["pi05_bf16_b1"]
    params, pk, pv, noise, state, _ = case(cfg)
    gu = _gu()
    got = run_stream(cfg, params, pk, pv, noise, state)
    per = gu.run_gpu(cfg, params, pk, pv, noise, state, "persistent")
    assert gu.rel_l2(got - noise, per - noise) <= TOL_DISP


def test_stream_zero_out_projection_keeps_noise_bitwise():
    cfg = tiny_bf16()
    params, pk, pv, noise, state = make_inputs(cfg)
    params["out_proj.w"] = np.zeros_like(params["out_proj.w"])
    params["out_proj.b"] = np.zeros_like(params["out_proj.b"])
    got = run_stream(cfg, params, pk, pv, noise, state)
    assert np.array_equal(got, noise)


def test_stream_constant_velocity_closed_form():
    """Zero out-projection weights and bias b: every Euler step moves the
    actions by -b / N, N steps give noise - b (in fp32: tolerance 1e-6)."""
    cfg = tiny_bf16()
    params, pk, pv, noise, state = make_inputs(cfg)
    vel = np.linspace(-1.5, 2.0, cfg.action_dim).astype(np.float32)
    params["out_proj.w"] = np.zeros_like(params["out_proj.w"])
    params["out_proj.b"] = vel
    got = run_stream(cfg, params, pk, pv, noise, state)
    np.testing.assert_allclose(got, noise.astype(np.float64) - vel, atol=1e-6, rtol=0)


def test_stream_unavailable_for_fp32_expert():
    from vla_flow_matching_pi0_amd import vfm
    gu = _gu()
    cfg = CONFIGS["tiny_fp32"]
    params, pk, pv, noise, state = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent")
    try:
        with pytest.raises(vfm.VfmError) as e:
            ex.set_option("launch_mode", "stream")
        assert "stream" in str(e.value)
        with pytest.raises(vfm.VfmError):
            ex.set_option("stream_dma_cap", "0")
    finally:
        ex.close()


def test_stream_rejects_batch_above_one():
    from vla_flow_matching_pi0_amd import vfm
    gu = _gu()
    cfg = tiny_bf16(batch=2)
    params, pk, pv, noise, state = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent", max_batch=2)
    try:
        ex.set_option("launch_mode", "stream")
        gu.bind_inputs(ex, cfg, pk, pv, noise, state)
        with pytest.raises(vfm.VfmError) as e:
            ex.denoise()
        assert "batch 1" in str(e.value)
    finally:
        ex.close()
