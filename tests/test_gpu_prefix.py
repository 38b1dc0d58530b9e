"""GPU parity of the prefix producer: the HIP pass through the C ABI against
the CPU float64 oracle (oracle/prefix.py) on the same seeded bf16 weights
and embeddings. The kernels round the GEMM inputs (normalised stream,
queries, attention output, GeGLU activations) and the outputs to bf16, so
the bar is relative L2 <= 2e-2 per layer for keys and values (the expert's
bf16 bar), with every element finite."""
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


def run_producer(cfg, params, emb, max_batch=None, max_prefix_len=None, producer=None):
    from vla_flow_matching_pi0_amd import vfm
    dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
    pre = producer or vfm.PrefixProducer(cfg, dev, max_batch=max_batch, max_prefix_len=max_prefix_len)
    del dev
    B, P = emb.shape[0], emb.shape[1]
    shape = (cfg.num_layers, B, P, cfg.num_kv_heads, cfg.head_dim)
    e = torch.from_numpy(emb).to("cuda").to(torch.bfloat16)
    pk = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    pv = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    pre.run(e, pk, pv)
    torch.cuda.synchronize()
    return pre, pk.float().cpu().numpy(), pv.float().cpu().numpy()


def check_layers(got_k, got_v, ref_k, ref_v, layers=None):
    assert np.isfinite(got_k).all() and np.isfinite(got_v).all()
    for l in (range(ref_k.shape[0]) if layers is None else layers):
        ek, ev = rel_l2(got_k[l], ref_k[l]), rel_l2(got_v[l], ref_v[l])
        print(f"layer {l}: k rel_l2 {ek:.3e}  v rel_l2 {ev:.3e}")
        assert ek <= TOL and ev <= TOL, l


def test_tiny_matches_oracle():
    cfg = PREFIX_CONFIGS["prefix_tiny"]
    params, emb = make_prefix_inputs(cfg)
    print("case prefix_tiny", flush=True)
    pre, k, v = run_producer(cfg, params, emb)
    pre.close()
    rk, rv = PO.prefix_kv(params, emb, cfg)
    check_layers(k, v, rk, rv)


@pytest.mark.parametrize("batch,prefix,heads", [(2, 37, (4, 1)), (3, 130, (4, 2)), (1, 1, (4, 1)), (1, 257, (8, 2))])
def test_ragged_shapes(batch, prefix, heads):
    """Batches whose token count is not a multiple of the 128-token tile,
    prefixes that are not a multiple of the 32-key tile, two KV heads."""
    cfg = PREFIX_CONFIGS["prefix_tiny"].replace(batch=batch, prefix_len=prefix, num_q_heads=heads[0],
                                                num_kv_heads=heads[1], seed=30 + prefix)
    params, emb = make_prefix_inputs(cfg)
    print(f"case prefix ragged B={batch} P={prefix} heads={heads}", flush=True)
    pre, k, v = run_producer(cfg, params, emb)
    pre.close()
    rk, rv = PO.prefix_kv(params, emb, cfg)
    check_layers(k, v, rk, rv)


@pytest.mark.parametrize("d", [128, 256])
def test_head_dims(d):
    cfg = PREFIX_CONFIGS["prefix_tiny"].replace(head_dim=d, num_q_heads=2, width=512, prefix_len=70, seed=40 + d)
    params, emb = make_prefix_inputs(cfg)
    print(f"case prefix d={d}", flush=True)
    pre, k, v = run_producer(cfg, params, emb)
    pre.close()
    rk, rv = PO.prefix_kv(params, emb, cfg)
    check_layers(k, v, rk, rv)


def test_rerun_with_other_shapes_on_one_producer():
    """One producer created for the largest shapes, run at a smaller batch and
    prefix and back (the rotary table and the tiling follow the call)."""
    cfg = PREFIX_CONFIGS["prefix_tiny"].replace(batch=2, prefix_len=90)
    params, emb = make_prefix_inputs(cfg)
    pre = None
    for b, P in ((2, 90), (1, 33), (2, 90)):
        c = cfg.replace(batch=b, prefix_len=P)
        e = np.ascontiguousarray(emb[:b, :P])
        pre, k, v = run_producer(c, params, e, max_batch=2, max_prefix_len=90, producer=pre)
        rk, rv = PO.prefix_kv(params, e, c)
        check_layers(k, v, rk, rv)
    pre.close()


@pytest.mark.parametrize("which", ["tiny_ragged", "gemma_two_layers"])
def test_gate_up_tiles_agree(which):
    """The gate/up GEMM on the 256-column tiles (the default where the shape
    takes them) and on the 128 x 128 tiles: both against the oracle per
    layer, and against each other: the same bf16 products summed in the
    same order and the same epilogue arithmetic, so the keys and values are
    bitwise equal (measured so on both shapes; asserted to 1e-3)."""
    from vla_flow_matching_pi0_amd import vfm
    if which == "tiny_ragged":   # 390 tokens: the last token tile ragged, tiles past the padded count
        cfg = PREFIX_CONFIGS["prefix_tiny"].replace(batch=3, prefix_len=130, seed=71)
    else:
        cfg = PREFIX_CONFIGS["prefix_gemma2b_p560"].replace(num_layers=2, seed=72)
    params, emb = make_prefix_inputs(cfg)
    rk, rv = PO.prefix_kv(params, emb, cfg)
    got = {}
    for tiles in ("narrow", "wide"):
        print(f"case prefix gate/up tiles {which} {tiles}", flush=True)
        dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
        pre = vfm.PrefixProducer(cfg, dev)
        del dev
        pre.set_option("gate_up_tiles", tiles)
        pre, k, v = run_producer(cfg, params, emb, producer=pre)
        pre.close()
        check_layers(k, v, rk, rv)
        got[tiles] = (k, v)
    for l in range(cfg.num_layers):
        ek = rel_l2(got["wide"][0][l], got["narrow"][0][l])
        ev = rel_l2(got["wide"][1][l], got["narrow"][1][l])
        print(f"layer {l}: wide vs narrow k {ek:.3e} v {ev:.3e}")
        assert ek <= 1e-3 and ev <= 1e-3, l


def test_down_tiles_agree():
    """The down projection on the 256-column tiles with 8 K splits (the
    default at the Gemma-2B shape, P = 560: 4 x 8 tiles x 8 splits) and on
    the 128 x 128 tiles with 4: both against the oracle per layer, and
    against each other to 1e-3 (the same products, partial sums added in
    another grouping). Layer 1's keys and values see layer 0's down
    projection through the residual stream."""
    from vla_flow_matching_pi0_amd import vfm
    cfg = PREFIX_CONFIGS["prefix_gemma2b_p560"].replace(num_layers=2, seed=73)
    params, emb = make_prefix_inputs(cfg)
    rk, rv = PO.prefix_kv(params, emb, cfg)
    got = {}
    for tiles in ("narrow", "wide"):
        print(f"case prefix down tiles {tiles}", flush=True)
        dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
        pre = vfm.PrefixProducer(cfg, dev)
        del dev
        pre.set_option("down_tiles", tiles)
        pre, k, v = run_producer(cfg, params, emb, producer=pre)
        pre.close()
        check_layers(k, v, rk, rv)
        got[tiles] = (k, v)
    for l in range(cfg.num_layers):
        ek = rel_l2(got["wide"][0][l], got["narrow"][0][l])
        ev = rel_l2(got["wide"][1][l], got["narrow"][1][l])
        print(f"layer {l}: wide vs narrow k {ek:.3e} v {ev:.3e}")
        assert ek <= 1e-3 and ev <= 1e-3, l


def test_qkv_tiles_bitwise_equal():
    """The fused QKV projection on 128 x 64 tiles (the default at the
    Gemma-2B shape: 100 tiles of 128 x 128 would leave most compute units
    idle) and on 128 x 128 tiles: every output is the same sum of the same
    bf16 products in the same k order, so the keys and values agree bit for
    bit; both match the oracle."""
    from vla_flow_matching_pi0_amd import vfm
    cfg = PREFIX_CONFIGS["prefix_gemma2b_p560"].replace(num_layers=2, seed=74)
    params, emb = make_prefix_inputs(cfg)
    rk, rv = PO.prefix_kv(params, emb, cfg)
    got = {}
    for tiles in ("full", "auto"):
        print(f"case prefix qkv tiles {tiles}", flush=True)
        dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
        pre = vfm.PrefixProducer(cfg, dev)
        del dev
        pre.set_option("qkv_tiles", tiles)
        pre, k, v = run_producer(cfg, params, emb, producer=pre)
        pre.close()
        check_layers(k, v, rk, rv)
        got[tiles] = (k, v)
    assert np.array_equal(got["full"][0], got["auto"][0]) and np.array_equal(got["full"][1], got["auto"][1])


def test_o_tiles_agree():
    """The o projection on 128 x 64 tiles with 2 K splits (the default at the
    Gemma-2B shape) and on 128 x 128 tiles with 4: both against the oracle
    per layer, and against each other to 1e-3 (the partial sums added in
    another grouping)."""
    from vla_flow_matching_pi0_amd import vfm
    cfg = PREFIX_CONFIGS["prefix_gemma2b_p560"].replace(num_layers=2, seed=75)
    params, emb = make_prefix_inputs(cfg)
    rk, rv = PO.prefix_kv(params, emb, cfg)
    got = {}
    for tiles in ("full", "auto"):
        print(f"case prefix o tiles {tiles}", flush=True)
        dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
        pre = vfm.PrefixProducer(cfg, dev)
        del dev
        pre.set_option("o_tiles", tiles)
        pre, k, v = run_producer(cfg, params, emb, producer=pre)
        pre.close()
        check_layers(k, v, rk, rv)
        got[tiles] = (k, v)
    for l in range(cfg.num_layers):
        ek = rel_l2(got["auto"][0][l], got["full"][0][l])
        ev = rel_l2(got["auto"][1][l], got["full"][1][l])
        print(f"layer {l}: half vs full o tiles k {ek:.3e} v {ev:.3e}")
        assert ek <= 1e-3 and ev <= 1e-3, l


def test_prefix_option_is_validated():
    from vla_flow_matching_pi0_amd import vfm
    cfg = PREFIX_CONFIGS["prefix_tiny"]
    params, _ = make_prefix_inputs(cfg)
    dev = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in params.items()}
    pre = vfm.PrefixProducer(cfg, dev)
    try:
        for key, val in (("gate_up_tiles", "huge"), ("down_tiles", "1"), ("qkv_tiles", "half"), ("o_tiles", "x"), ("no_such_option", "1")):
            with pytest.raises(vfm.VfmError) as e:
                pre.set_option(key, val)
            assert e.value.name == "VFM_E_INVALID_ARG"
    finally:
        pre.close()


def test_gemma_shape_three_layers():
    """Every kernel at the Gemma-2B per-layer shape (width 2048, 8 query heads
    sharing one KV head of dim 256, GeGLU 16384, 560 prefix tokens: the
    launch configuration the benchmark times per layer), at depth 3."""
    cfg = PREFIX_CONFIGS["prefix_gemma2b_p560"].replace(num_layers=3)
    params, emb = make_prefix_inputs(cfg)
    print("case prefix gemma2b shape, 3 layers", flush=True)
    pre, k, v = run_producer(cfg, params, emb)
    pre.close()
    rk, rv = PO.prefix_kv(params, emb, cfg)
    check_layers(k, v, rk, rv)


def test_producer_feeds_the_expert():
    """The chain the pages describe: prefix pass, then the action expert's
    denoise loop on the keys and values it wrote (device buffers handed over
    without a copy), against the oracle chain."""
    from vla_flow_matching_pi0_amd import vfm
    import gpu_util as gu
    pcfg = PREFIX_CONFIGS["prefix_tiny"].replace(prefix_len=64, batch=2)
    ecfg = CONFIGS["tiny_fp32"].replace(weight_precision="bf16", batch=2, prefix_len=64, state_dim=4,
                                        num_layers=pcfg.num_layers, num_kv_heads=pcfg.num_kv_heads,
                                        head_dim=pcfg.head_dim)
    pparams, emb = make_prefix_inputs(pcfg)
    eparams, _, _, noise, state = make_inputs(ecfg)
    print("case prefix -> expert chain", flush=True)
    pre = vfm.PrefixProducer(pcfg, {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in pparams.items()})
    shape = (pcfg.num_layers, 2, 64, pcfg.num_kv_heads, pcfg.head_dim)
    pk = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    pv = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    ex = gu.build_expert(ecfg, eparams)
    bufs = gu.bind_inputs(ex, ecfg, np.zeros(shape, np.float32), np.zeros(shape, np.float32), noise, state)
    ex.bind("prefix_k", pk)
    ex.bind("prefix_v", pv)
    pre.run(torch.from_numpy(emb).to("cuda").to(torch.bfloat16), pk, pv)
    ex.denoise()
    ex.check()
    torch.cuda.synchronize()
    got = bufs["actions"].cpu().numpy()
    rk, rv = PO.prefix_kv(pparams, emb, pcfg)
    ref = O.denoise(eparams, noise, state, rk, rv, ecfg)
    err = rel_l2(got, ref)
    print(f"chain: actions rel_l2 {err:.3e}")
    assert err <= TOL
    pre.close()
    ex.close()


def test_full_depth_every_layer():
    """The full 18-layer Gemma-2B-shaped pass at 560 tokens (what the benchmark
    times): every layer's keys and values against the fp64 oracle element-wise
    (the whole-depth oracle pass, about a minute on the host)."""
    cfg = PREFIX_CONFIGS["prefix_gemma2b_p560"]
    params, emb = make_prefix_inputs(cfg)
    print("case prefix gemma2b full depth", flush=True)
    pre, k, v = run_producer(cfg, params, emb)
    pre.close()
    rk, rv = PO.prefix_kv(params, emb, cfg)
    check_layers(k, v, rk, rv)
