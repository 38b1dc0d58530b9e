"""Build libvfm.so (the HIP kernels for gfx950 and the C ABI runtime) in-tree.

Usage: python -m vla_flow_matching_pi0_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvfm.so")
SOURCES = ["vfm_k_bf16.hip", "vfm_k_attn.hip", "vfm_k_fp8.hip", "vfm_k_w4.hip", "vfm_k_i8.hip", "vfm_k_w4a8.hip", "vfm_k_cal.hip", "vfm_k_stream.hip", "vfm_k_f32.hip", "vfm_prep.hip",
           "vfm_prefix.hip", "vfm_launch.cpp", "vfm_runtime.cpp", "vfm_stream_rt.cpp", "vfm_prefix_rt.cpp", "vfm_plan.cpp"]

# per-file additions: the large-batch attention keeps its MFMA accumulators
# in VGPRs (it rescales them with vector ALU operations between MFMAs)
EXTRA_FLAGS = {"vfm_k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libvfm.so; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), *inc, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and "warning generated" not in l)
        if p.returncode != 0:
            failed.append(f"{src}:\n{out}")
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("HIP build failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
