"""GPU parity of the pi0 variant (state token, action-time MLP, plain norms,
the state token's attention limited to the prefix and itself) through the C
ABI against the CPU float64 oracle (oracle/pi0.py). Bars: relative L2
1e-4 (fp32), 2e-2 (bf16) on the final actions."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pi0 as P0
from synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_pi0_amd import vfm
    vfm.load_library()


def _gu():
    import gpu_util
    return gpu_util


@pytest.mark.parametrize("mode", ["persistent", "graph", "eager"])
def test_pi0_tiny_fp32_matches_oracle(mode):
    gu = _gu()
    cfg = CONFIGS["pi0_tiny_fp32"]
    params, pk, pv, noise, state = make_inputs(cfg)
    print(f"case pi0 tiny mode={mode}", flush=True)
    got = gu.run_gpu(cfg, params, pk, pv, noise, state, mode)
    ref = P0.denoise_pi0(params, noise, state, pk, pv, cfg)
    err = gu.rel_l2(got, ref)
    disp = gu.rel_l2(got - noise, ref - noise)
    print(f"pi0 tiny {mode}: rel_l2={err:.3e} displacement rel_l2={disp:.3e}")
    assert err <= 1e-4
    assert disp <= 1e-3


@pytest.mark.parametrize("batch,prefix,horizon", [(2, 37, 13), (3, 5, 1), (1, 130, 63)])
def test_pi0_ragged_shapes(batch, prefix, horizon):
    """Batches, prefixes off the 64-key split, horizons that leave 1 to 64
    suffix tokens (the largest fills the 64-token tile with the state token)."""
    gu = _gu()
    cfg = CONFIGS["pi0_tiny_fp32"].replace(batch=batch, prefix_len=prefix, action_horizon=horizon, seed=40 + horizon)
    params, pk, pv, noise, state = make_inputs(cfg)
    print(f"case pi0 ragged B={batch} P={prefix} H={horizon}", flush=True)
    got = gu.run_gpu(cfg, params, pk, pv, noise, state, "persistent")
    ref = P0.denoise_pi0(params, noise, state, pk, pv, cfg)
    err = gu.rel_l2(got, ref)
    print(f"pi0 ragged: rel_l2={err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("mode", ["persistent", "graph"])
def test_pi0_bf16_b1_matches_oracle(mode):
    gu = _gu()
    cfg = CONFIGS["pi0_bf16_b1"]
    params, pk, pv, noise, state = make_inputs(cfg)
    print(f"case pi0 bf16 mode={mode}", flush=True)
    got = gu.run_gpu(cfg, params, pk, pv, noise, state, mode)
    ref = P0.denoise_pi0(params, noise, state, pk, pv, cfg)
    # measured 2.6e-3 / 1.5e-2: the displacement error is forty times the
    # pi0.5 expert's at the same precision (an open item); bounds at about
    # three times the measurement
    gu.assert_parity(got, ref, noise, 1e-2, 5e-2, 1e-1, f"pi0 bf16 {mode}")


def test_pi0_state_changes_the_actions_and_the_trace_has_two_more_barriers_per_step():
    """The state reaches the actions only through the state token (so a
    different state gives other actions, matching the oracle), and the
    persistent kernel runs 6 barriers per layer (the attention merge in place) plus 3 per step."""
    gu = _gu()
    cfg = CONFIGS["pi0_tiny_fp32"].replace(num_steps=3)
    params, pk, pv, noise, state = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent")
    ex.set_option("trace", "1")
    bufs = gu.bind_inputs(ex, cfg, pk, pv, noise, state)
    plan = ex.persistent_plan()
    ex.denoise()
    ex.check()
    a1 = bufs["actions"].cpu().numpy()
    L, N = cfg.num_layers, cfg.num_steps
    t = ex.export("trace", (2 * (N * (8 * L + 3) + 4),)).reshape(-1, 2)
    n_bar = plan["barriers"]
    assert plan["attn_merge"] and n_bar == 1 + N * (6 * L + 2)
    stamps = t[1:n_bar + 1].ravel()
    assert np.all(stamps >= 0) and np.all(np.diff(stamps) >= 0)
    state2 = state + 1.0
    bufs["state"].copy_(torch.from_numpy(state2))
    ex.denoise()
    ex.check()
    torch.cuda.synchronize()
    a2 = bufs["actions"].cpu().numpy()
    ex.close()
    assert np.abs(a1 - a2).max() > 1e-4
    assert gu.rel_l2(a2, P0.denoise_pi0(params, noise, state2, pk, pv, cfg)) <= 1e-4
