"""ctypes binding of libvfm.so (include/vfm.h).

Argument marshalling only: every step of the denoise loop runs in the HIP
kernels of the library. PyTorch supplies device memory and streams. There is
no fallback: if the library is missing or a call fails, an exception says so.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Mapping, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvfm.so")

VFM_F32, VFM_BF16, VFM_F16, VFM_FP8_E4M3, VFM_I4X2 = 0, 1, 2, 3, 4
WPREC = {"fp32": 0, "bf16": 1, "fp8": 2, "w4a16": 3, "w8a16": 4, "w4a8": 5}
VARIANT = {"pi05": 0, "pi0": 1}
STATUS = {0: "VFM_OK", 1: "VFM_E_INVALID_ARG", 2: "VFM_E_SHAPE", 3: "VFM_E_DTYPE", 4: "VFM_E_UNBOUND",
          5: "VFM_E_STATE", 6: "VFM_E_UNSUPPORTED", 7: "VFM_E_OOM", 8: "VFM_E_HIP"}
ABI_VERSION = 2

# Every entry point include/vfm.h declares.
EXPORTS = ["vfm_abi_version", "vfm_last_error", "vfm_expert_create", "vfm_bind", "vfm_denoise",
           "vfm_set_option", "vfm_calibrate", "vfm_set_act_scales", "vfm_export", "vfm_copy_probe", "vfm_check",
           "vfm_expert_destroy", "vfm_stream_debug", "vfm_capsule_create", "vfm_capsule_save", "vfm_capsule_restore",
           "vfm_capsule_bytes", "vfm_capsule_destroy", "vfm_prefix_create", "vfm_prefix_run",
           "vfm_prefix_run_noalloc", "vfm_prefix_set_option", "vfm_prefix_destroy", "vfm_plan_create", "vfm_plan_add_prefix", "vfm_plan_add_denoise",
           "vfm_plan_add_graph", "vfm_plan_add_edge", "vfm_plan_deps", "vfm_plan_run", "vfm_plan_destroy"]


class VfmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class VfmConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "num_layers", "width", "num_q_heads", "num_kv_heads", "head_dim", "mlp_dim",
        "action_horizon", "action_dim", "state_dim", "time_emb_dim", "max_prefix_len", "max_batch",
        "num_steps")] + [("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float),
                         ("weight_precision", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                         ("w4_group_size", ctypes.c_int32), ("variant", ctypes.c_int32)]


class VfmPrefixConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "num_layers", "width", "num_q_heads", "num_kv_heads", "head_dim", "mlp_dim",
        "max_prefix_len", "max_batch")] + [("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class VfmRange(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("bytes", ctypes.c_size_t)]


class VfmTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dev_ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 4)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvfm.so and declare the signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m vla_flow_matching_pi0_amd.build`")
    # torch brings its own HIP runtime; load it first so that the library binds
    # to the same runtime as the tensors it is handed (two runtimes in one
    # process do not share device allocations)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.vfm_abi_version.restype = ctypes.c_int
    lib.vfm_last_error.restype = ctypes.c_char_p
    lib.vfm_expert_create.argtypes = [ctypes.POINTER(VfmConfig), ctypes.POINTER(VfmTensor), i32, vp,
                                      ctypes.POINTER(vp)]
    lib.vfm_bind.argtypes = [vp, ctypes.c_char_p, vp, i32, i32, ctypes.POINTER(ctypes.c_int64)]
    lib.vfm_denoise.argtypes = [vp, vp, vp, vp, vp]
    lib.vfm_stream_debug.argtypes = [vp, ctypes.c_char_p, i32, vp, ctypes.c_size_t]
    lib.vfm_set_option.argtypes = [vp, ctypes.c_char_p, ctypes.c_char_p]
    lib.vfm_calibrate.argtypes = [vp, vp]
    lib.vfm_set_act_scales.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32]
    lib.vfm_export.argtypes = [vp, ctypes.c_char_p, vp, ctypes.c_size_t]
    lib.vfm_check.argtypes = [vp, vp]
    lib.vfm_copy_probe.argtypes = [vp, vp, ctypes.c_size_t, i32, vp]
    lib.vfm_expert_destroy.argtypes = [vp]
    lib.vfm_capsule_create.argtypes = [vp, ctypes.POINTER(vp)]
    lib.vfm_capsule_save.argtypes = [vp, vp, vp]
    lib.vfm_capsule_restore.argtypes = [vp, vp, vp]
    lib.vfm_capsule_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.vfm_capsule_destroy.argtypes = [vp]
    lib.vfm_prefix_create.argtypes = [ctypes.POINTER(VfmPrefixConfig), ctypes.POINTER(VfmTensor), i32, vp,
                                      ctypes.POINTER(vp)]
    lib.vfm_prefix_run.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.vfm_prefix_run_noalloc.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.vfm_prefix_set_option.argtypes = [vp, ctypes.c_char_p, ctypes.c_char_p]
    lib.vfm_prefix_destroy.argtypes = [vp]
    lib.vfm_plan_create.argtypes = [ctypes.POINTER(vp)]
    lib.vfm_plan_add_prefix.argtypes = [vp, vp, vp, i32, i32, vp, vp, i32, i32, ctypes.POINTER(i32)]
    lib.vfm_plan_add_denoise.argtypes = [vp, vp, vp, vp, vp, i32, i32, ctypes.POINTER(i32)]
    lib.vfm_plan_add_graph.argtypes = [vp, vp, ctypes.POINTER(VfmRange), i32, ctypes.POINTER(VfmRange), i32, i32, i32,
                                       ctypes.POINTER(i32)]
    lib.vfm_plan_add_edge.argtypes = [vp, i32, i32]
    lib.vfm_plan_deps.argtypes = [vp, ctypes.c_int64, i32, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]
    lib.vfm_plan_run.argtypes = [vp, ctypes.c_int64, vp]
    lib.vfm_plan_destroy.argtypes = [vp]
    for n in EXPORTS[2:]:
        getattr(lib, n).restype = st
    if lib.vfm_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libvfm ABI {lib.vfm_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = _lib.vfm_last_error().decode(errors="replace")
        raise VfmError(status, msg)


def make_config(cfg, max_batch: Optional[int] = None, max_prefix_len: Optional[int] = None) -> VfmConfig:
    """Build the C config from any object with the expert's fields
    (num_layers, width, ..., weight_precision in WPREC, variant 'pi05' or 'pi0')."""
    c = VfmConfig()
    c.abi_version = ABI_VERSION
    for n in ("num_layers", "width", "num_q_heads", "num_kv_heads", "head_dim", "mlp_dim", "action_horizon",
              "action_dim", "state_dim", "time_emb_dim", "num_steps"):
        setattr(c, n, int(getattr(cfg, n)))
    c.max_prefix_len = int(max_prefix_len if max_prefix_len is not None else cfg.prefix_len)
    c.max_batch = int(max_batch if max_batch is not None else cfg.batch)
    c.rope_base = float(cfg.rope_base)
    c.rms_eps = float(cfg.rms_eps)
    c.weight_precision = WPREC[cfg.weight_precision]
    c.act_dtype = VFM_F32 if cfg.weight_precision == "fp32" else VFM_BF16
    c.w4_group_size = int(getattr(cfg, "w4_group", 128))
    c.variant = VARIANT[getattr(cfg, "variant", "pi05")]
    return c


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: VFM_F32, torch.bfloat16: VFM_BF16, torch.float16: VFM_F16}[t.dtype]


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class Expert:
    """One action expert living on the current HIP device.

    weights: name -> device tensor (row-major [in][out]); fp32 for fp32
    experts, bf16 otherwise. They may be freed once the constructor returns."""

    def __init__(self, cfg, weights: Mapping[str, "object"], stream=None, max_batch: Optional[int] = None,
                 max_prefix_len: Optional[int] = None):
        lib = load_library()
        self._cfg = cfg
        self._ccfg = make_config(cfg, max_batch, max_prefix_len)
        names = list(weights.keys())
        arr = (VfmTensor * len(names))()
        self._names = [n.encode() for n in names]
        for i, n in enumerate(names):
            t = weights[n]
            arr[i].name = self._names[i]
            arr[i].dev_ptr = t.data_ptr()
            arr[i].dtype = _dtype_code(t)
            arr[i].ndim = t.dim()
            for j, s in enumerate(t.shape):
                arr[i].shape[j] = int(s)
        h = ctypes.c_void_p()
        _check(lib.vfm_expert_create(ctypes.byref(self._ccfg), arr, len(names), _stream_ptr(stream), ctypes.byref(h)))
        self._h = h
        self._bound: Dict[str, object] = {}

    # -------------------------------------------------------------- buffers
    def bind(self, name: str, t) -> None:
        shape = (ctypes.c_int64 * t.dim())(*[int(s) for s in t.shape])
        _check(_lib.vfm_bind(self._h, name.encode(), t.data_ptr(), _dtype_code(t), t.dim(), shape))
        self._bound[name] = t            # keep the memory alive while bound

    def set_option(self, key: str, value: str) -> None:
        _check(_lib.vfm_set_option(self._h, key.encode(), value.encode()))

    def denoise(self, noise=None, state=None, out=None, stream=None):
        """Run the loop; returns `out` (or the bound actions buffer)."""
        ptr = lambda t: None if t is None else t.data_ptr()
        _check(_lib.vfm_denoise(self._h, ptr(noise), ptr(state), ptr(out), _stream_ptr(stream)))
        return out if out is not None else self._bound.get("actions")

    def check(self, stream=None) -> None:
        _check(_lib.vfm_check(self._h, _stream_ptr(stream)))

    def calibrate(self, stream=None) -> None:
        _check(_lib.vfm_calibrate(self._h, _stream_ptr(stream)))

    def set_act_scales(self, scales) -> None:
        a = np.ascontiguousarray(scales, dtype=np.float32)
        _check(_lib.vfm_set_act_scales(self._h, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), a.size))

    def export(self, name: str, shape) -> np.ndarray:
        out = np.empty(shape, dtype=np.float32)
        _check(_lib.vfm_export(self._h, name.encode(), out.ctypes.data, out.nbytes))
        return out

    def persistent_plan(self) -> dict:
        """The persistent kernel's plan at the bound batch and prefix (vfm_export "persistent_plan")."""
        out = np.empty(6, dtype=np.int32)
        _check(_lib.vfm_export(self._h, b"persistent_plan", out.ctypes.data, out.nbytes))
        return {"fused_norms": bool(out[0]), "barriers": int(out[1]), "o_splits": int(out[2]), "down_splits": int(out[3]),
                "xcd_local": bool(out[4]), "attn_merge": bool(out[5])}

    def stream_debug(self, name: str, index: int = 0, nbytes: int = 0) -> np.ndarray:
        """Raw bytes of an internal buffer of the streaming kernel (diagnostics; see vfm_stream_debug)."""
        if name == "slab_layout":
            out = np.empty(10, dtype=np.uint64)
        else:
            out = np.empty(nbytes, dtype=np.uint8)
        _check(_lib.vfm_stream_debug(self._h, name.encode(), index, out.ctypes.data, out.nbytes))
        return out

    def capsule(self) -> "Capsule":
        """A capsule sized for the current bindings (holds no state until saved)."""
        return Capsule(self)

    def close(self) -> None:
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            _check(_lib.vfm_expert_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Capsule:
    """Snapshot of an expert's bound buffers (and FP8 activation scales):
    save() and restore() enqueue device-to-device copies on a stream;
    restore() into another expert of the same layout forks the state."""

    def __init__(self, expert: Expert):
        h = ctypes.c_void_p()
        _check(_lib.vfm_capsule_create(expert._h, ctypes.byref(h)))
        self._h = h

    def save(self, expert: Expert, stream=None) -> None:
        _check(_lib.vfm_capsule_save(expert._h, self._h, _stream_ptr(stream)))

    def restore(self, expert: Expert, stream=None) -> None:
        _check(_lib.vfm_capsule_restore(expert._h, self._h, _stream_ptr(stream)))

    @property
    def nbytes(self) -> int:
        n = ctypes.c_size_t()
        _check(_lib.vfm_capsule_bytes(self._h, ctypes.byref(n)))
        return n.value

    def close(self) -> None:
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            _check(_lib.vfm_capsule_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_prefix_config(cfg, max_batch: Optional[int] = None, max_prefix_len: Optional[int] = None) -> VfmPrefixConfig:
    """C config of the prefix producer from any object with its fields."""
    c = VfmPrefixConfig()
    c.abi_version = ABI_VERSION
    for n in ("num_layers", "width", "num_q_heads", "num_kv_heads", "head_dim", "mlp_dim"):
        setattr(c, n, int(getattr(cfg, n)))
    c.max_prefix_len = int(max_prefix_len or cfg.prefix_len)
    c.max_batch = int(max_batch or cfg.batch)
    c.rope_base = float(cfg.rope_base)
    c.rms_eps = float(cfg.rms_eps)
    return c


def _tensor_array(weights):
    names = list(weights.keys())
    arr = (VfmTensor * len(names))()
    keep = [n.encode() for n in names]
    for i, n in enumerate(names):
        t = weights[n]
        arr[i].name = keep[i]
        arr[i].dev_ptr = t.data_ptr()
        arr[i].dtype = _dtype_code(t)
        arr[i].ndim = t.dim()
        for j, sz in enumerate(t.shape):
            arr[i].shape[j] = int(sz)
    return arr, keep


class PrefixProducer:
    """The vision + language prefix pass that writes the per-layer prefix K/V
    an Expert binds. weights: name -> bf16 device tensor."""

    def __init__(self, cfg, weights: Mapping[str, "object"], stream=None, max_batch: Optional[int] = None,
                 max_prefix_len: Optional[int] = None):
        lib = load_library()
        self._ccfg = make_prefix_config(cfg, max_batch, max_prefix_len)
        arr, keep = _tensor_array(weights)
        h = ctypes.c_void_p()
        _check(lib.vfm_prefix_create(ctypes.byref(self._ccfg), arr, len(keep), _stream_ptr(stream), ctypes.byref(h)))
        self._h = h

    def run(self, embeds, prefix_k, prefix_v, stream=None) -> None:
        """embeds [B][P][W] bf16 -> prefix_k, prefix_v [L][B][P][Hkv][d] bf16 (all device tensors)."""
        B, P = int(embeds.shape[0]), int(embeds.shape[1])
        _check(_lib.vfm_prefix_run(self._h, embeds.data_ptr(), B, P, prefix_k.data_ptr(), prefix_v.data_ptr(),
                                   _stream_ptr(stream)))

    def run_noalloc(self, embeds, prefix_k, prefix_v, stream=None) -> None:
        """run() with the workspace in the library's static per-device array (no allocation)."""
        B, P = int(embeds.shape[0]), int(embeds.shape[1])
        _check(_lib.vfm_prefix_run_noalloc(self._h, embeds.data_ptr(), B, P, prefix_k.data_ptr(),
                                           prefix_v.data_ptr(), _stream_ptr(stream)))

    def set_option(self, key: str, value: str) -> None:
        _check(_lib.vfm_prefix_set_option(self._h, key.encode(), value.encode()))

    def close(self) -> None:
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            _check(_lib.vfm_prefix_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr(t) -> Optional[int]:
    """Device address of a tensor, an int address, or None (NULL)."""
    if t is None:
        return None
    return t if isinstance(t, int) else t.data_ptr()


def _ranges(items):
    """(tensor | (address, bytes)) list -> C array of vfm_range."""
    arr = (VfmRange * max(1, len(items)))()
    for i, it in enumerate(items):
        if isinstance(it, tuple):
            arr[i].ptr, arr[i].bytes = int(it[0]), int(it[1])
        else:
            arr[i].ptr, arr[i].bytes = it.data_ptr(), it.numel() * it.element_size()
    return arr


class Plan:
    """Stages (prefix passes, denoise calls, adopted graphs) with update
    rates; dependencies are derived from the buffers each stage reads and
    writes. run(tick) enqueues the due stages on their own streams, forked
    from and joined into the caller's stream. Keeps references to everything
    its stages point at."""

    def __init__(self):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.vfm_plan_create(ctypes.byref(h)))
        self._h = h
        self._keep = []

    def add_prefix(self, producer: PrefixProducer, embeds, prefix_k, prefix_v, every: int = 1,
                   offset: int = 0) -> int:
        sid = ctypes.c_int32()
        _check(_lib.vfm_plan_add_prefix(self._h, producer._h, embeds.data_ptr(), int(embeds.shape[0]),
                                        int(embeds.shape[1]), prefix_k.data_ptr(), prefix_v.data_ptr(), every, offset,
                                        ctypes.byref(sid)))
        self._keep += [producer, embeds, prefix_k, prefix_v]
        return sid.value

    def add_denoise(self, expert: Expert, noise=None, state=None, actions=None, every: int = 1,
                    offset: int = 0) -> int:
        sid = ctypes.c_int32()
        _check(_lib.vfm_plan_add_denoise(self._h, expert._h, _ptr(noise), _ptr(state), _ptr(actions), every, offset,
                                         ctypes.byref(sid)))
        self._keep += [expert, noise, state, actions]
        return sid.value

    def add_graph(self, graph_exec, reads=(), writes=(), every: int = 1, offset: int = 0) -> int:
        """graph_exec: an int hipGraphExec_t, or a torch.cuda.CUDAGraph
        (its executable graph is adopted; the CUDAGraph must stay alive)."""
        h = graph_exec if isinstance(graph_exec, int) else graph_exec.raw_cuda_graph_exec()
        r, w = list(reads), list(writes)
        sid = ctypes.c_int32()
        _check(_lib.vfm_plan_add_graph(self._h, h, _ranges(r), len(r), _ranges(w), len(w), every, offset,
                                       ctypes.byref(sid)))
        self._keep += [graph_exec, *r, *w]
        return sid.value

    def add_edge(self, src: int, dst: int) -> None:
        _check(_lib.vfm_plan_add_edge(self._h, src, dst))

    def deps(self, tick: int, stage: int):
        """Stages that `stage` waits for at `tick`, or None if it does not run then."""
        buf = (ctypes.c_int32 * 256)()
        n = ctypes.c_int32()
        _check(_lib.vfm_plan_deps(self._h, tick, stage, buf, 256, ctypes.byref(n)))
        return None if n.value < 0 else [buf[i] for i in range(n.value)]

    def run(self, tick: int, stream=None) -> None:
        _check(_lib.vfm_plan_run(self._h, tick, _stream_ptr(stream)))

    def close(self) -> None:
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            _check(_lib.vfm_plan_destroy(h))
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def copy_probe(src, dst, policy: int, stream=None) -> None:
    """Measurement helper: copy src -> dst (device tensors of equal byte size)
    with loads of cache policy 0 (plain), 1 (sc0) or 16 (sc1)."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    _check(lib.vfm_copy_probe(src.data_ptr(), dst.data_ptr(), nbytes, policy, _stream_ptr(stream)))
