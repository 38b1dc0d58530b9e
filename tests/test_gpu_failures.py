"""Failure reporting through the C ABI, forced from the host.

Option "fail_barrier" makes one device-wide barrier wait for one arrival more
than the grid holds; "barrier_spin_limit" bounds that wait, so it gives up
after about a millisecond and every workgroup exits normally (no kernel is
left waiting). The failure must surface as VFM_E_HIP from vfm_check even when
a second call, which itself would have succeeded, was queued behind the
failed one before anything synchronised (the error word is sticky: no launch
clears it, only the host after reporting it). Once reported, the expert runs
correctly again."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import denoise as O
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


@pytest.mark.parametrize("mode", ["persistent", "stream"])
def test_barrier_timeout_is_reported_after_a_queued_call(mode):
    from vla_flow_matching_pi0_amd import vfm
    gu = _gu()
    cfg = CONFIGS["tiny_fp32"].replace(weight_precision="bf16", state_dim=8) if mode == "stream" else CONFIGS["tiny_fp32"]
    params, pk, pv, noise, state = make_inputs(cfg)
    ref = O.denoise(params, noise, state, pk, pv, cfg)
    ex = gu.build_expert(cfg, params, mode)
    try:
        bufs = gu.bind_inputs(ex, cfg, pk, pv, noise, state)
        ex.set_option("barrier_spin_limit", "4096")
        ex.set_option("fail_barrier", "3")
        print(f"case {mode}: failing call, then a good call queued behind it", flush=True)
        ex.denoise()
        ex.set_option("fail_barrier", "0")
        # the failure surfaces exactly once: from the second call if the first
        # had already finished when it was enqueued, else from vfm_check
        errors = []
        for call in (ex.denoise, ex.check):
            try:
                call()
            except vfm.VfmError as err:
                errors.append(err)
        assert len(errors) == 1, errors
        assert errors[0].name == "VFM_E_HIP"
        assert "timed out" in str(errors[0])
        # reported once; the expert works again
        ex.check()
        ex.denoise()
        ex.check()
        torch.cuda.synchronize()
        got = bufs["actions"].cpu().numpy()
        tol = 1e-4 if mode == "persistent" else 2e-3
        assert gu.rel_l2(got, ref) <= tol
    finally:
        ex.close()


def test_failure_options_are_validated():
    from vla_flow_matching_pi0_amd import vfm
    gu = _gu()
    cfg = CONFIGS["tiny_fp32"]
    params, pk, pv, noise, state = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent")
    try:
        for key, val in [("barrier_spin_limit", "10"), ("barrier_spin_limit", "x"), ("fail_barrier", "-1")]:
            with pytest.raises(vfm.VfmError) as e:
                ex.set_option(key, val)
            assert e.value.name == "VFM_E_INVALID_ARG"
    finally:
        ex.close()
