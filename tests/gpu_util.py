"""Helpers for the GPU parity tests: move the seeded synthetic inputs onto
the device and run the library through its C ABI binding."""
from __future__ import annotations

import numpy as np
import torch

from synth import make_inputs
from vla_flow_matching_pi0_amd import vfm


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def device_params(cfg, params):
    dt = torch.float32 if cfg.master_dtype == "f32" else torch.bfloat16
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(dt) for k, v in params.items()}


def build_expert(cfg, params, mode="persistent", max_batch=None, max_prefix_len=None):
    ex = vfm.Expert(cfg, device_params(cfg, params), max_batch=max_batch, max_prefix_len=max_prefix_len)
    ex.set_option("launch_mode", mode)
    return ex


def bind_inputs(ex, cfg, pk, pv, noise, state):
    adt = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16
    bufs = {
        "prefix_k": torch.from_numpy(pk).to("cuda").to(adt).contiguous(),
        "prefix_v": torch.from_numpy(pv).to("cuda").to(adt).contiguous(),
        "noise": torch.from_numpy(noise).to("cuda").contiguous(),
        "actions": torch.empty(noise.shape, dtype=torch.float32, device="cuda"),
    }
    if cfg.state_dim > 0:
        bufs["state"] = torch.from_numpy(state).to("cuda").contiguous()
    for k, v in bufs.items():
        ex.bind(k, v)
    return bufs


def run_gpu(cfg, params, pk, pv, noise, state, mode="persistent", repeats=1):
    ex = build_expert(cfg, params, mode)
    bufs = bind_inputs(ex, cfg, pk, pv, noise, state)
    for _ in range(repeats):
        ex.denoise()
    ex.check()
    torch.cuda.synchronize()
    out = bufs["actions"].cpu().numpy()
    ex.close()
    return out


def inputs(cfg):
    return make_inputs(cfg)


def parity_errors(got, ref, noise):
    """(relative L2 of the actions, relative L2 of the displacement actions -
    noise, largest element error of the displacement relative to the largest
    reference displacement)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    noise = np.asarray(noise, dtype=np.float64)
    d_got, d_ref = got - noise, ref - noise
    elem = float(np.max(np.abs(d_got - d_ref)) / np.max(np.abs(d_ref)))
    return rel_l2(got, ref), rel_l2(d_got, d_ref), elem


def assert_parity(got, ref, noise, rel, disp, elem, label=""):
    """Assert the three parity errors against their bounds (and print them)."""
    e = parity_errors(got, ref, noise)
    print(f"{label}: rel_l2={e[0]:.3e} displacement rel_l2={e[1]:.3e} max element {e[2]:.3e}", flush=True)
    assert np.isfinite(np.asarray(got)).all(), label
    assert e[0] <= rel, (label, "rel_l2", e[0])
    assert e[1] <= disp, (label, "displacement", e[1])
    assert e[2] <= elem, (label, "element", e[2])
