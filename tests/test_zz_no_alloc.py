"""vfm_prefix_run_noalloc (the prefix pass with its workspace in the
library's static per-device array) against vfm_prefix_run on the same
producer and inputs: the results must be identical, for two calls in a row
where the second is smaller than the first (so it runs over what the first
left in the array), and a call whose workspace exceeds the array fails
cleanly. The keys and values are also checked against the fp64 oracle at the
prefix tests' bar (relative L2 2e-2 per layer)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import prefix as PO
from synth import PREFIX_CONFIGS, make_prefix_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_pi0_amd import vfm
    vfm.load_library()


def _outputs(cfg, B, P):
    shape = (cfg.num_layers, B, P, cfg.num_kv_heads, cfg.head_dim)
    return (torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda"))


def _rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_noalloc_matches_run_on_two_calls_the_second_smaller():
    from vla_flow_matching_pi0_amd import vfm
    base = PREFIX_CONFIGS["prefix_tiny"]
    calls = [base.replace(batch=2, prefix_len=100), base.replace(batch=1, prefix_len=37)]
    params, _ = make_prefix_inputs(calls[0])
    dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
    pre = vfm.PrefixProducer(base, dev, max_batch=2, max_prefix_len=100)
    del dev
    try:
        for i, cfg in enumerate(calls):
            _, emb = make_prefix_inputs(cfg)
            B, P = emb.shape[0], emb.shape[1]
            print(f"call {i}: batch {B} prefix {P}", flush=True)
            e = torch.from_numpy(emb).to("cuda").to(torch.bfloat16)
            k1, v1 = _outputs(cfg, B, P)
            k2, v2 = _outputs(cfg, B, P)
            pre.run_noalloc(e, k1, v1)
            pre.run(e, k2, v2)
            torch.cuda.synchronize()
            a_k, a_v = k1.float().cpu().numpy(), v1.float().cpu().numpy()
            b_k, b_v = k2.float().cpu().numpy(), v2.float().cpu().numpy()
            assert np.isfinite(a_k).all() and np.isfinite(a_v).all()
            assert np.array_equal(a_k, b_k) and np.array_equal(a_v, b_v)
            ref_k, ref_v = PO.prefix_kv(params, emb, cfg)
            for l in range(cfg.num_layers):
                assert _rel_l2(a_k[l], ref_k[l]) <= 2e-2 and _rel_l2(a_v[l], ref_v[l]) <= 2e-2, (i, l)
    finally:
        pre.close()


def test_noalloc_rejects_a_workspace_beyond_the_static_array():
    from vla_flow_matching_pi0_amd import vfm
    cfg = PREFIX_CONFIGS["prefix_tiny"]
    params, _ = make_prefix_inputs(cfg)
    dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
    # 16 x 2048 tokens of width 256: about 140 MB of workspace, beyond 64 MiB
    pre = vfm.PrefixProducer(cfg, dev, max_batch=16, max_prefix_len=2048)
    del dev
    try:
        e = torch.zeros((16, 2048, cfg.width), dtype=torch.bfloat16, device="cuda")
        k, v = _outputs(cfg, 16, 2048)
        with pytest.raises(vfm.VfmError) as err:
            pre.run_noalloc(e, k, v)
        assert err.value.name == "VFM_E_UNSUPPORTED"
        assert "static workspace" in str(err.value)
    finally:
        pre.close()
