"""Host-side checks of bench.py (no GPU): the algorithmic byte and FLOP
counts behind the roofline against the shapes written out by hand, the
choice of roofline per workload, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bytes_per_step_pi05_bf16():
    """18 layers of q/k/v (1024 x 10 x 256), o (2048 x 1024), gate/up
    (2 x 1024 x 4096) and down (4096 x 1024) in bf16, in/out projections
    (2 x 32 x 1024), and the prefix K and V (2 x 18 x 560 x 256): 622.99 MB
    of weights and 10.32 MB of prefix per Euler step; the state projection
    (32 x 1024) once per call."""
    cfg = CONFIGS["pi05_bf16_b1"]
    weights = 18 * (1024 * 2560 + 2048 * 1024 + 2 * 1024 * 4096 + 4096 * 1024) * 2 + 2 * 32 * 1024 * 2
    prefix = 2 * 18 * 560 * 256 * 2
    assert weights == 622_985_216 and prefix == 10_321_920
    assert bench.algorithmic_bytes_per_step(cfg) == weights + prefix
    assert bench.algorithmic_bytes_per_launch(cfg) == 10 * (weights + prefix) + 32 * 1024 * 2
    assert abs(bench.algorithmic_bytes_per_launch(cfg) / 8e12 * 1e3 - 0.7917) < 1e-3   # ms at 8 TB/s


def test_quantised_and_batched_bytes():
    b1 = CONFIGS["pi05_bf16_b1"]
    per_layer = 1024 * 2560 + 2048 * 1024 + 2 * 1024 * 4096 + 4096 * 1024
    io = 2 * 32 * 1024 * 2
    # W4A16: a nibble per weight plus an fp16 scale per 128 weights
    w4 = CONFIGS["pi05_w4a16"]
    assert bench.algorithmic_bytes_per_step(w4) == 18 * (per_layer // 2 + per_layer // 128 * 2) + io + 2 * 18 * 560 * 256 * 2
    # batch 32: the same weights, 32 prefixes
    b32 = CONFIGS["pi05_bf16_b32"]
    assert bench.algorithmic_bytes_per_step(b32) - bench.algorithmic_bytes_per_step(b1) == 31 * 2 * 18 * 560 * 256 * 2


def test_flops_per_chunk():
    """2 x multiply-adds of the GEMMs and attention: about 356 GFLOP per batch-1
    chunk and 11.41 TFLOP per batch-32 chunk."""
    assert abs(bench.flops_per_chunk(CONFIGS["pi05_bf16_b1"]) / 356e9 - 1) < 0.01
    assert abs(bench.flops_per_chunk(CONFIGS["pi05_bf16_b32"]) / 11.41e12 - 1) < 0.01


def test_roofline_bound_per_workload():
    """Batch 1 streams weights (HBM-bound in every format); batch 32 needs
    4.6 ms of bf16 MFMA work against 1.2 ms of bytes (MFMA-bound)."""
    for name in ("pi05_bf16_b1", "pi05_fp8_p816", "pi05_w4a16", "pi05_w8a16", "pi05_w4a8", "pi0_bf16_b1"):
        assert bench.roofline_bound(CONFIGS[name]) == "hbm", name
    assert bench.roofline_bound(CONFIGS["pi05_bf16_b32"]) == "mfma"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_auto_mode_resolution_matches_the_library_rule():
    assert bench.resolved_mode(CONFIGS["pi05_bf16_b1"], "auto") == "persistent"
    assert bench.resolved_mode(CONFIGS["pi05_bf16_b32"], "auto") == "graph"
    assert bench.resolved_mode(CONFIGS["pi05_fp8_p816"], "auto") == "persistent"
    assert bench.resolved_mode(CONFIGS["pi05_bf16_b32"], "eager") == "eager"


def _timeline(N, L, fused, merged, work, wait):
    """(arrive, release) stamps of workgroup 0 for the persistent kernel's
    phase sequence, each phase taking work[name] before its barrier and
    wait[name] at it: the boundary, then per Euler step every layer's phases
    (separate norms: layer l > 0 starts with rn_attn, layer 0's norm is in
    the boundary) and the step boundary."""
    import numpy as np
    if fused:
        layer = lambda l: ["qkv_attn", "o", "gu", "down"]
    elif merged:
        layer = lambda l: (["rn_attn"] if l else []) + ["qkv_attn", "o", "rn_mlp", "gu", "down"]
    else:
        layer = lambda l: (["rn_attn"] if l else []) + ["qkv", "attn", "combine", "o", "rn_mlp", "gu", "down"]
    seq = ["boundary"]
    for _ in range(N):
        for l in range(L):
            seq += layer(l)
        seq.append("boundary")
    t = np.zeros((len(seq) + 1, 2))
    now = 0.0
    for i, name in enumerate(seq):
        now += work.get(name, 1.0)
        t[i + 1, 0] = now
        now += wait.get(name, 0.5)
        t[i + 1, 1] = now
    return t, len(seq)


@pytest.mark.parametrize("fused,merged", [(True, True), (False, True), (False, False)])
def test_phase_breakdown_recovers_each_phase(fused, merged):
    """bench.phase_breakdown reads a middle layer's (work, wait) per phase
    from the barrier timeline: on a synthetic timeline with a distinct
    duration per phase it returns those durations, for the folded-norm
    kernel (4 barriers per layer + 1 per step), the separate-norm kernel
    with the in-place merge (6 per layer) and with the combine phase (8)."""
    N, L = 3, 5
    names = (["qkv_attn", "o", "gu", "down"] if fused
             else ["rn_attn", "qkv_attn", "o", "rn_mlp", "gu", "down"] if merged
             else ["rn_attn", "qkv", "attn", "combine", "o", "rn_mlp", "gu", "down"])
    work = {n: 2.0 + i for i, n in enumerate(names)}
    wait = {n: 0.25 * (i + 1) for i, n in enumerate(names)}
    t, nb = _timeline(N, L, fused, merged, work, wait)
    assert nb == (1 + N * (4 * L + 1) if fused else 1 + N * ((6 if merged else 8) * L))
    got = bench.phase_breakdown(t, nb, N, L, fused, 0, merged)
    assert set(got) == set(names)
    for n in names:
        assert got[n] == [round(work[n], 2), round(wait[n], 2)], n
