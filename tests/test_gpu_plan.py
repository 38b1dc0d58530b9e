"""GPU tests of plans (vfm_plan_*) and of the expert's graph variant table.

Every tick's actions are compared with the oracle chain (oracle/prefix.py
for the prefix K/V, oracle/denoise.py for the loop) on the inputs that tick
should have seen: with a prefix stage refreshing every third tick, the ticks
in between must use the K/V of the last refresh even when the embeddings
buffer already holds the next observation. Bar: relative L2 <= 2e-2 (bf16
weights, K/V and activations), as for the producer -> expert chain."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import denoise as O
from oracle import prefix as PO
from synth import CONFIGS, PREFIX_CONFIGS, make_inputs, make_prefix_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_pi0_amd import vfm
    vfm.load_library()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def bf16_grid(x):
    return torch.from_numpy(np.asarray(x, np.float32)).bfloat16().float().numpy()


@pytest.fixture(scope="module")
def chain():
    """Producer + expert configs and weights of the tiny chain (prefix 64,
    batch 2), two observations, and the oracle K/V of each."""
    pcfg = PREFIX_CONFIGS["prefix_tiny"].replace(prefix_len=64, batch=2)
    ecfg = CONFIGS["tiny_fp32"].replace(weight_precision="bf16", batch=2, prefix_len=64, state_dim=4,
                                        num_layers=pcfg.num_layers, num_kv_heads=pcfg.num_kv_heads,
                                        head_dim=pcfg.head_dim)
    pparams, emb_a = make_prefix_inputs(pcfg)
    emb_b = bf16_grid(np.random.default_rng(77).standard_normal(emb_a.shape))
    eparams, _, _, _, state = make_inputs(ecfg)
    kv = {"a": PO.prefix_kv(pparams, emb_a, pcfg), "b": PO.prefix_kv(pparams, emb_b, pcfg)}
    return dict(pcfg=pcfg, ecfg=ecfg, pparams=pparams, eparams=eparams, emb={"a": emb_a, "b": emb_b}, kv=kv,
                state=state)


def dev(x, dt=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dt)


def make_producer(c):
    from vla_flow_matching_pi0_amd import vfm
    return vfm.PrefixProducer(c["pcfg"], {k: dev(v, torch.bfloat16) for k, v in c["pparams"].items()})


def make_expert(c, mode, pk, pv, state):
    from vla_flow_matching_pi0_amd import vfm
    ex = vfm.Expert(c["ecfg"], {k: dev(v, torch.bfloat16) for k, v in c["eparams"].items()})
    ex.set_option("launch_mode", mode)
    ex.bind("prefix_k", pk)
    ex.bind("prefix_v", pv)
    ex.bind("state", state)
    return ex


def kv_buffers(c):
    p = c["pcfg"]
    shape = (p.num_layers, p.batch, p.prefix_len, p.num_kv_heads, p.head_dim)
    return (torch.empty(shape, dtype=torch.bfloat16, device="cuda"),
            torch.empty(shape, dtype=torch.bfloat16, device="cuda"))


def noise_for(tick, shape, salt=0):
    return np.random.default_rng(1000 * salt + tick).standard_normal(shape).astype(np.float32)


def expect(c, obs, noise):
    rk, rv = c["kv"][obs]
    return O.denoise(c["eparams"], noise, c["state"], rk, rv, c["ecfg"])


@pytest.mark.parametrize("mode", ["graph", "persistent"])
def test_selective_refresh_every_third_tick(chain, mode):
    """Prefix stage every 3 ticks, expert every tick. The next observation is
    written into the embeddings buffer at tick 1, but the prefix is refreshed
    only at tick 3: ticks 1 and 2 must still act on the first observation."""
    from vla_flow_matching_pi0_amd import vfm
    c = chain
    print(f"case plan selective refresh, {mode} expert", flush=True)
    emb = dev(c["emb"]["a"], torch.bfloat16)
    pk, pv = kv_buffers(c)
    state = dev(c["state"])
    shape = (c["ecfg"].batch, c["ecfg"].action_horizon, c["ecfg"].action_dim)
    noise = torch.empty(shape, dtype=torch.float32, device="cuda")
    actions = torch.empty_like(noise)
    pre = make_producer(c)
    ex = make_expert(c, mode, pk, pv, state)
    ex.bind("noise", noise)
    ex.bind("actions", actions)
    plan = vfm.Plan()
    sp = plan.add_prefix(pre, emb, pk, pv, every=3)
    se = plan.add_denoise(ex)
    assert plan.deps(0, se) == [sp] and plan.deps(1, se) == [] and plan.deps(1, sp) is None
    seen = {0: "a", 1: "a", 2: "a", 3: "b", 4: "b", 5: "b"}
    for t in range(6):
        if t == 1:
            emb.copy_(dev(c["emb"]["b"], torch.bfloat16))
        n = noise_for(t, shape)
        noise.copy_(dev(n))
        plan.run(t)
        got = actions.cpu().numpy()
        err = rel_l2(got, expect(c, seen[t], n))
        print(f"tick {t}: observation {seen[t]}, actions rel_l2 {err:.3e}")
        assert err <= TOL, t
    ex.check()
    plan.close()
    ex.close()
    pre.close()


def test_fork_two_experts_share_one_prefix(chain):
    """Two graph-mode experts with their own noise read the K/V one prefix
    stage wrote: each waits for the prefix stage only (they run side by side
    on their own streams); a persistent-mode expert waits for all three; a
    second stage on the same expert waits for the first."""
    from vla_flow_matching_pi0_amd import vfm
    c = chain
    print("case plan fork", flush=True)
    emb = dev(c["emb"]["a"], torch.bfloat16)
    pk, pv = kv_buffers(c)
    state = dev(c["state"])
    shape = (c["ecfg"].batch, c["ecfg"].action_horizon, c["ecfg"].action_dim)
    pre = make_producer(c)
    e1, e2 = make_expert(c, "graph", pk, pv, state), make_expert(c, "graph", pk, pv, state)
    e3 = make_expert(c, "persistent", pk, pv, state)
    noise = [torch.empty(shape, dtype=torch.float32, device="cuda") for _ in range(4)]
    acts = [torch.empty_like(noise[0]) for _ in range(4)]
    plan = vfm.Plan()
    sp = plan.add_prefix(pre, emb, pk, pv)
    s1 = plan.add_denoise(e1, noise=noise[0], actions=acts[0])
    s2 = plan.add_denoise(e2, noise=noise[1], actions=acts[1])
    s3 = plan.add_denoise(e3, noise=noise[2], actions=acts[2])
    s4 = plan.add_denoise(e1, noise=noise[3], actions=acts[3])
    assert plan.deps(0, s1) == [sp] and plan.deps(0, s2) == [sp]
    assert plan.deps(0, s3) == [sp, s1, s2]
    assert plan.deps(0, s4) == [sp, s1, s3]
    for t, obs in ((0, "a"), (1, "b")):
        emb.copy_(dev(c["emb"][obs], torch.bfloat16))
        ns = [noise_for(t, shape, salt=i + 1) for i in range(4)]
        for buf, n in zip(noise, ns):
            buf.copy_(dev(n))
        plan.run(t)
        for i in range(4):
            err = rel_l2(acts[i].cpu().numpy(), expect(c, obs, ns[i]))
            print(f"tick {t} stage {i + 1}: rel_l2 {err:.3e}")
            assert err <= TOL, (t, i)
    for e in (e1, e2, e3):
        e.check()
    plan.close()
    for e in (e1, e2, e3):
        e.close()
    pre.close()


def test_adopted_torch_graph_feeds_the_expert(chain):
    """A torch-captured graph (noise = 0.5 * staging buffer) adopted as a stage
    ahead of the expert: the expert waits for it, and each tick's actions
    follow the staging buffer written on the caller's stream before the
    tick. The adopted graph is replayed at every tick, with host copies and
    synchronisations between replays."""
    from vla_flow_matching_pi0_amd import vfm
    c = chain
    print("case plan adopted torch graph", flush=True)
    rk, rv = c["kv"]["a"]
    pk, pv = dev(rk, torch.bfloat16), dev(rv, torch.bfloat16)
    state = dev(c["state"])
    shape = (c["ecfg"].batch, c["ecfg"].action_horizon, c["ecfg"].action_dim)
    staging = torch.zeros(shape, dtype=torch.float32, device="cuda")
    noise = torch.zeros_like(staging)
    actions = torch.empty_like(staging)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.mul(staging, 0.5, out=noise)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        torch.mul(staging, 0.5, out=noise)
    torch.cuda.synchronize()
    ex = make_expert(c, "persistent", pk, pv, state)
    ex.bind("noise", noise)
    ex.bind("actions", actions)
    plan = vfm.Plan()
    sg = plan.add_graph(graph, reads=[staging], writes=[noise])
    se = plan.add_denoise(ex)
    assert plan.deps(0, se) == [sg]
    pk_oracle, pv_oracle = pk.float().cpu().numpy(), pv.float().cpu().numpy()
    for t in range(3):
        raw = noise_for(t, shape, salt=9)
        staging.copy_(dev(raw))
        plan.run(t)
        torch.cuda.synchronize()
        got = actions.cpu().numpy()
        np.testing.assert_array_equal(noise.cpu().numpy(), 0.5 * raw)
        ref = O.denoise(c["eparams"], 0.5 * raw, c["state"], pk_oracle, pv_oracle, c["ecfg"])
        err = rel_l2(got, ref)
        print(f"tick {t}: rel_l2 {err:.3e}")
        assert err <= TOL, t
    ex.check()
    plan.close()
    ex.close()


@pytest.mark.parametrize("cache", [1, 8])
def test_graph_variants_alternate_shapes_and_buffers(chain, cache):
    """Graph mode with two prefix lengths and two noise / actions pairs,
    alternated: with room for both variants the second round replays the
    cached graphs (the rotary table of the other length is rebuilt in place
    before each), with one slot every call captures again. Both must match
    the oracle on every call."""
    c = chain
    print(f"case graph variants, cache {cache}", flush=True)
    ecfg = c["ecfg"]
    _, pk_np, pv_np, _, _ = make_inputs(ecfg)
    state = dev(c["state"])
    shape = (ecfg.batch, ecfg.action_horizon, ecfg.action_dim)
    kv = {64: (pk_np, pv_np), 40: (np.ascontiguousarray(pk_np[:, :, :40]), np.ascontiguousarray(pv_np[:, :, :40]))}
    kv_dev = {P: (dev(k, torch.bfloat16), dev(v, torch.bfloat16)) for P, (k, v) in kv.items()}
    ns = [noise_for(0, shape, salt=20), noise_for(1, shape, salt=20)]
    noise = [dev(n) for n in ns]
    acts = [torch.empty_like(noise[0]) for _ in range(2)]
    ex = make_expert(c, "graph", *kv_dev[64], state)
    ex.set_option("graph_cache", str(cache))
    for rnd in range(2):
        for i, P in enumerate((64, 40)):
            ex.bind("prefix_k", kv_dev[P][0])
            ex.bind("prefix_v", kv_dev[P][1])
            ex.denoise(noise=noise[i], out=acts[i])
            got = acts[i].cpu().numpy()
            kb = bf16_grid(kv[P][0].astype(np.float32))
            vb = bf16_grid(kv[P][1].astype(np.float32))
            ref = O.denoise(c["eparams"], ns[i], c["state"], kb, vb, ecfg.replace(prefix_len=P))
            err = rel_l2(got, ref)
            print(f"round {rnd} P={P}: rel_l2 {err:.3e}")
            assert err <= TOL, (rnd, P)
    ex.check()
    ex.close()


def test_unbound_stage_is_refused_before_anything_runs(chain):
    """A tick whose denoise stage lacks its prefix binding fails on the host
    with VFM_E_UNBOUND before any stage is enqueued: the prefix stage ahead of
    it leaves its outputs untouched. Binding the buffers makes the same tick
    run."""
    from vla_flow_matching_pi0_amd import vfm
    c = chain
    print("case plan unbound stage", flush=True)
    emb = dev(c["emb"]["a"], torch.bfloat16)
    pk, pv = kv_buffers(c)
    pk.fill_(7.0)
    pv.fill_(7.0)
    pre = make_producer(c)
    ex = vfm.Expert(c["ecfg"], {k: dev(v, torch.bfloat16) for k, v in c["eparams"].items()})
    shape = (c["ecfg"].batch, c["ecfg"].action_horizon, c["ecfg"].action_dim)
    noise = dev(noise_for(0, shape, salt=30))
    actions = torch.zeros_like(noise)
    plan = vfm.Plan()
    plan.add_prefix(pre, emb, pk, pv)
    se = plan.add_denoise(ex, noise=noise, state=dev(c["state"]), actions=actions)
    with pytest.raises(vfm.VfmError) as e:
        plan.run(0)
    assert e.value.name == "VFM_E_UNBOUND"
    with pytest.raises(vfm.VfmError):
        plan.deps(0, se)
    torch.cuda.synchronize()
    assert bool((pk.float() == 7.0).all()) and bool((actions == 0).all())
    ex.bind("prefix_k", pk)
    ex.bind("prefix_v", pv)
    ex.bind("state", dev(c["state"]))
    plan.run(0)
    err = rel_l2(actions.cpu().numpy(), expect(c, "a", noise.cpu().numpy()))
    print(f"after binding: rel_l2 {err:.3e}")
    assert err <= TOL
    plan.close()
    ex.close()
    pre.close()
