"""GPU parity of the persistent kernel with the adaptive RMSNorms folded into
the GEMMs (option "fused_norms", bf16 pi0.5 experts): against the fp64
oracle and against the same kernel with separate norm phases, on the
pi0.5 batch-1 workload, ragged and multi-tile shapes, K splits of the o and
down projections with and without the last-arriver epilogue, repeated calls
and a change of batch between calls (the split counters must start every
launch at zero whatever the previous launch split).

The folded form computes xn W as r (y W) + shift W with y = h (1 + scale)
rounded to bf16 instead of xn, so the two variants differ by bf16 rounding
of the GEMM inputs: the bounds are those of the bf16 parity tests (relative
L2 2e-3, displacement 5e-3, element 1e-2 on the batch-1 workload; 2e-2 on
the actions elsewhere), and fused against unfused within the same."""
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


def _run(cfg, params, pk, pv, noise, state, fused, repeats=1, plain=False, xcd_local=True):
    gu = _gu()
    ex = gu.build_expert(cfg, params, "persistent")
    ex.set_option("fused_norms", "1" if fused else "0")
    ex.set_option("xcd_local", "1" if xcd_local else "0")
    if plain:
        ex.set_option("persistent_launch", "plain")
    bufs = gu.bind_inputs(ex, cfg, pk, pv, noise, state)
    plan = ex.persistent_plan()
    for _ in range(repeats):
        bufs["actions"].fill_(float("nan"))
        ex.denoise()
    ex.check()
    torch.cuda.synchronize()
    out = bufs["actions"].cpu().numpy()
    ex.close()
    return out, plan


def test_pi05_b1_fused_matches_oracle_and_unfused():
    gu = _gu()
    cfg = CONFIGS["pi05_bf16_b1"].replace(num_layers=4)
    params, pk, pv, noise, state = make_inputs(cfg)
    ref = O.denoise(params, noise, state, pk, pv, cfg)
    print("case pi05 b1 (4 layers) fused / unfused", flush=True)
    fused, pf = _run(cfg, params, pk, pv, noise, state, True, repeats=3)
    plain, pp = _run(cfg, params, pk, pv, noise, state, False)
    L, N = cfg.num_layers, cfg.num_steps
    assert pf["fused_norms"] and not pp["fused_norms"]
    assert pf["barriers"] == 1 + N * (4 * L + 1) and pp["barriers"] == 1 + N * 6 * L
    assert pf["o_splits"] > 1 and pf["down_splits"] > 1   # the last-arriver epilogue runs
    gu.assert_parity(fused, ref, noise, 2e-3, 5e-3, 1e-2, "fused")
    gu.assert_parity(plain, ref, noise, 2e-3, 5e-3, 1e-2, "unfused")
    gu.assert_parity(fused, plain, noise, 2e-3, 5e-3, 1e-2, "fused vs unfused")


@pytest.mark.parametrize("shape", [
    # several 64-row tiles with a ragged last one (M = 150), two layers
    dict(num_layers=2, batch=3, prefix_len=37),
    # a horizon that is not a multiple of 16, one layer (only o's residual is folded; the step boundary
    # finishes down's)
    dict(num_layers=1, batch=2, action_horizon=13, prefix_len=70),
    # width 256: one sums-of-squares load per lane, head dim 64, GQA
    dict(num_layers=2, width=256, num_q_heads=4, num_kv_heads=2, head_dim=64, mlp_dim=512, time_emb_dim=256,
         action_horizon=20, action_dim=8, state_dim=3, prefix_len=50, batch=1),
    # width 512 at batch 5: 250 rows
    dict(num_layers=2, width=512, num_q_heads=8, num_kv_heads=1, head_dim=128, mlp_dim=1024, time_emb_dim=512,
         prefix_len=33, batch=5),
])
def test_fused_shapes_match_oracle(shape):
    gu = _gu()
    cfg = CONFIGS["pi05_bf16_b1"].replace(**shape)
    params, pk, pv, noise, state = make_inputs(cfg)
    ref = O.denoise(params, noise, state, pk, pv, cfg)
    print(f"case fused shape {shape}", flush=True)
    fused, pf = _run(cfg, params, pk, pv, noise, state, True, repeats=2)
    plain, _ = _run(cfg, params, pk, pv, noise, state, False)
    print(f"plan {pf}")
    assert pf["fused_norms"]
    e_f, e_p, e_fp = gu.rel_l2(fused, ref), gu.rel_l2(plain, ref), gu.rel_l2(fused, plain)
    print(f"fused rel_l2={e_f:.3e} unfused {e_p:.3e} fused vs unfused {e_fp:.3e}")
    assert np.isfinite(fused).all()
    assert e_f <= 2e-2 and e_p <= 2e-2 and e_fp <= 2e-2


def test_batch_change_between_fused_calls():
    """One expert, calls at batch 1 (4-way K splits of o and down), batch 4
    (no splits) and batch 1 again: each matches the oracle."""
    gu = _gu()
    cfg = CONFIGS["pi05_bf16_b1"].replace(num_layers=2, batch=4, prefix_len=40)
    params, pk, pv, noise, state = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent", max_batch=4)
    ex.set_option("fused_norms", "1")   # batch 4 (200 rows) folds only when asked to
    splits = []
    for b in (1, 4, 1):
        c = cfg.replace(batch=b)
        bufs = gu.bind_inputs(ex, c, pk[:, :b].copy(), pv[:, :b].copy(), noise[:b].copy(), state[:b].copy())
        plan = ex.persistent_plan()
        assert plan["fused_norms"]
        splits.append(plan["o_splits"])
        print(f"case batch {b} plan {plan}", flush=True)
        for _ in range(2):
            ex.denoise()
        ex.check()
        torch.cuda.synchronize()
        got = bufs["actions"].cpu().numpy()
        ref = O.denoise(params, noise[:b], state[:b], pk[:, :b], pv[:, :b], c)
        err = gu.rel_l2(got, ref)
        print(f"batch {b}: rel_l2={err:.3e}")
        assert err <= 2e-2, b
    ex.close()
    assert splits[0] != splits[1]   # the split count did change between the calls


def test_fused_plain_launch_and_trace():
    """The ordinary launch of the fused kernel and its phase timeline: the
    number of barriers the plan states, each released after it was reached
    and before the next is reached."""
    gu = _gu()
    cfg = CONFIGS["pi05_bf16_b1"].replace(num_layers=2, num_steps=3)
    params, pk, pv, noise, state = make_inputs(cfg)
    ref = O.denoise(params, noise, state, pk, pv, cfg)
    ex = gu.build_expert(cfg, params, "persistent")
    ex.set_option("persistent_launch", "plain")
    ex.set_option("trace", "1")
    bufs = gu.bind_inputs(ex, cfg, pk, pv, noise, state)
    plan = ex.persistent_plan()
    ex.denoise()
    ex.check()
    torch.cuda.synchronize()
    assert gu.rel_l2(bufs["actions"].cpu().numpy(), ref) <= 2e-2
    L, N = cfg.num_layers, cfg.num_steps
    # the trace buffer also fits the streaming kernel's timeline (3 words per barrier)
    words = max(2 * (N * (8 * L + 1) + 4), 3 * (N * (5 * L + 2) + 1))
    t = ex.export("trace", (words,))[: 2 * (N * (8 * L + 1) + 4)].reshape(-1, 2)
    ex.close()
    nb = plan["barriers"]
    assert nb == 1 + N * (4 * L + 1)
    stamps = t[1:nb + 1].ravel()
    assert np.all(stamps >= 0) and np.all(np.diff(stamps) >= 0)


def test_fused_norms_auto_folds_small_calls_only():
    """The default ("auto") folds the norms for calls of at most 128 rows
    (pi0.5 batch 1 and 2); larger calls run separate norm phases unless
    "1" asks for the folded kernel."""
    gu = _gu()
    cfg = CONFIGS["pi05_bf16_b1"].replace(num_layers=2, batch=32, prefix_len=40)
    params, pk, pv, noise, state = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent", max_batch=32)
    got = {}
    for b in (1, 2, 4, 32):
        bufs = gu.bind_inputs(ex, cfg.replace(batch=b), pk[:, :b].copy(), pv[:, :b].copy(), noise[:b].copy(), state[:b].copy())
        got[b] = ex.persistent_plan()["fused_norms"]
    ex.set_option("fused_norms", "1")
    forced = ex.persistent_plan()["fused_norms"]
    ex.close()
    print(f"auto fold by batch {got}, batch 32 with '1': {forced}")
    assert got == {1: True, 2: True, 4: False, 32: False}
    assert forced


def test_fused_norms_option_is_validated():
    from vla_flow_matching_pi0_amd import vfm
    gu = _gu()
    cfg = CONFIGS["tiny_fp32"]
    params, *_ = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent")
    with pytest.raises(vfm.VfmError) as e:
        ex.set_option("fused_norms", "1")
    assert e.value.name == "VFM_E_UNSUPPORTED"
    ex.set_option("fused_norms", "0")
    ex.set_option("fused_norms", "auto")
    with pytest.raises(vfm.VfmError) as e:
        ex.set_option("fused_norms", "yes")
    assert e.value.name == "VFM_E_INVALID_ARG"
    ex.close()


def test_xcd_local_split_sums_bitwise_equal_device_path():
    """The o / down split sums exchanged through one XCD's L2 (the default)
    against the device-coherence-point exchange: the same products summed in
    the same split order, so the actions agree bit for bit, over several
    calls (the XCD-local counters carry over between launches); both match
    the oracle."""
    gu = _gu()
    cfg = CONFIGS["pi05_bf16_b1"].replace(num_layers=4, num_steps=4)
    params, pk, pv, noise, state = make_inputs(cfg)
    ref = O.denoise(params, noise, state, pk, pv, cfg)
    print("case pi05 b1 (4 layers, 4 steps) xcd_local 1 / 0", flush=True)
    loc, pl = _run(cfg, params, pk, pv, noise, state, True, repeats=3)
    dev, pd = _run(cfg, params, pk, pv, noise, state, True, repeats=3, xcd_local=False)
    print(f"plans {pl} {pd}")
    assert pl["xcd_local"] and not pd["xcd_local"]
    assert pl["o_splits"] > 1 and pl["down_splits"] > 1
    assert np.array_equal(loc, dev)
    gu.assert_parity(loc, ref, noise, 2e-3, 5e-3, 1e-2, "xcd-local")


def test_xcd_local_option_is_validated():
    from vla_flow_matching_pi0_amd import vfm
    gu = _gu()
    cfg = CONFIGS["tiny_fp32"]
    params, *_ = make_inputs(cfg)
    ex = gu.build_expert(cfg, params, "persistent")
    with pytest.raises(vfm.VfmError) as e:
        ex.set_option("xcd_local", "2")
    assert e.value.name == "VFM_E_INVALID_ARG"
    ex.set_option("xcd_local", "0")
    ex.close()


@pytest.mark.parametrize("prec", ["w4a16", "w8a16"])
def test_weight_only_quantised_fused_matches_oracle_and_unfused(prec):
    """Weight-only quantised experts (bf16 activations) take the folded-norm
    kernel too, with shift W tables built from the weights the GEMMs
    multiply by (bf16 (q s) for int4, codes times column scales for int8):
    against the oracle on the dequantised expert and against the same
    expert with separate norm phases."""
    from oracle import quant as Q
    gu = _gu()
    cfg = CONFIGS["pi05_" + prec].replace(num_layers=4)
    params, pk, pv, noise, state = make_inputs(cfg)
    deq, _ = Q.dequantised_expert(params, cfg)
    ref = O.denoise(deq, noise, state, pk, pv, cfg)
    print(f"case {prec} (4 layers) fused / unfused", flush=True)
    fused, pf = _run(cfg, params, pk, pv, noise, state, True, repeats=2)
    plain, pp = _run(cfg, params, pk, pv, noise, state, False)
    assert pf["fused_norms"] and not pp["fused_norms"]
    gu.assert_parity(fused, ref, noise, 2e-3, 5e-3, 1e-2, f"{prec} fused")
    gu.assert_parity(fused, plain, noise, 2e-3, 5e-3, 1e-2, f"{prec} fused vs unfused")


@pytest.mark.parametrize("cfgname", ["pi05_bf16_b1", "pi0_tiny_fp32"])
def test_attn_merge_option_matches_combine_phase(cfgname):
    """The persistent kernel's in-place attention merge (default) against the
    combine phase between device-wide barriers (option attn_merge 0, which
    also selects separate norm phases): the same split outputs merged in the
    same order, so the actions agree to the folded-norm bound (bitwise where
    the norms are separate in both)."""
    gu = _gu()
    cfg = CONFIGS[cfgname]
    if cfgname == "pi05_bf16_b1":
        cfg = cfg.replace(num_layers=3, num_steps=3)
    params, pk, pv, noise, state = make_inputs(cfg)
    outs, plans = {}, {}
    for merge in ("1", "0"):
        for fused in ("1", "0"):
            if fused == "1" and (merge == "0" or cfgname != "pi05_bf16_b1"):
                continue
            print(f"case {cfgname} attn_merge={merge} fused_norms={fused}", flush=True)
            ex = gu.build_expert(cfg, params, "persistent")
            if cfgname == "pi05_bf16_b1":
                ex.set_option("fused_norms", fused)
            ex.set_option("attn_merge", merge)
            bufs = gu.bind_inputs(ex, cfg, pk, pv, noise, state)
            plans[(merge, fused)] = ex.persistent_plan()
            for _ in range(2):
                ex.denoise()
            ex.check()
            torch.cuda.synchronize()
            outs[(merge, fused)] = bufs["actions"].cpu().numpy()
            ex.close()
    assert plans[("1", "0")]["attn_merge"] and not plans[("0", "0")]["attn_merge"]
    assert not plans[("0", "0")]["fused_norms"]
    assert np.array_equal(outs[("1", "0")], outs[("0", "0")])
    if ("1", "1") in outs:
        assert plans[("1", "1")]["fused_norms"]
        gu.assert_parity(outs[("1", "1")], outs[("0", "0")], noise, 2e-3, 5e-3, 1e-2, "merged fused vs combine")
