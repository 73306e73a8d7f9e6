"""Thin Python binding of ``include/dit.h`` (ctypes).

Argument marshalling only: every step of the forward runs in ``libdit.so``.
torch supplies device memory (``torch.empty(..., device='cuda')``) and the
stream (``torch.cuda.current_stream()``).  torch is imported before the library
is loaded so both use the one HIP runtime already in the process.

The library is required: if ``libdit.so`` is missing this module raises at
import time instead of falling back to anything.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime first)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdit.so")

DIT_OK = 0
STATUS = {0: "DIT_OK", 1: "DIT_E_INVALID", 2: "DIT_E_STATE", 3: "DIT_E_UNKNOWN_WEIGHT", 4: "DIT_E_SHAPE",
          5: "DIT_E_DTYPE", 6: "DIT_E_MISSING_WEIGHT", 7: "DIT_E_WORKSPACE", 8: "DIT_E_HIP", 9: "DIT_E_UNSUPPORTED"}
DIT_F32, DIT_BF16, DIT_F64, DIT_MXFP8, DIT_MXFP4 = 0, 1, 2, 3, 4
DIT_GEMM_STREAM, DIT_GEMM_MXFP8, DIT_GEMM_MXFP4 = 0, 1, 2
DIT_NORM_RMS, DIT_NORM_LAYER = 0, 1
DIT_MLP_GATE_UP, DIT_MLP_VALUE_GATE = 0, 1
DIT_IO_NONE, DIT_IO_PATCH3D, DIT_IO_CHANNEL_MAJOR = 0, 1, 2
MAX_MOD = 4
COUNTER_NAMES = ["gemm_bf16", "gemm_f32", "attention_bf16", "attention_f32", "modnorm", "rope_split",
                 "silu_gate", "gated_residual", "adaln", "patch_in", "patch_out", "euler",
                 "gemm_f32_reduce", "convert", "resid_norm_slice", "silu_slice", "cfg_euler",
                 "resid_modnorm", "gemm_mx8", "quantize_mx8", "gemm_mx4", "quantize_mx4"]


class DitError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class dit_modality(ctypes.Structure):
    _fields_ = [("io", ctypes.c_int), ("channels", ctypes.c_int), ("patch", ctypes.c_int * 3),
                ("n_axes", ctypes.c_int), ("axis_dim", ctypes.c_int * 3), ("rope_grid", ctypes.c_int)]


class dit_config(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int), ("hidden", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int), ("norm", ctypes.c_int),
                ("norm_eps", ctypes.c_float), ("mlp", ctypes.c_int), ("rot_dim", ctypes.c_int),
                ("theta", ctypes.c_double), ("stream_dtype", ctypes.c_int), ("cond_dim", ctypes.c_int),
                ("n_mod", ctypes.c_int), ("io", ctypes.c_int), ("mod", dit_modality * MAX_MOD),
                ("gemm_format", ctypes.c_int), ("qkv_layout", ctypes.c_int), ("qk_norm", ctypes.c_int)]


class dit_segment(ctypes.Structure):
    _fields_ = [("modality", ctypes.c_int), ("cond_row", ctypes.c_int), ("grid", ctypes.c_int * 3)]


class dit_weight_view(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int), ("ndim", ctypes.c_int),
                ("shape", ctypes.c_int64 * 4), ("host", ctypes.c_void_p)]


class dit_stage_stats_t(ctypes.Structure):
    _fields_ = [("tensors", ctypes.c_int64), ("bytes", ctypes.c_int64), ("direct", ctypes.c_int64),
                ("converted", ctypes.c_int64), ("host_peak", ctypes.c_int64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "dit_pack_layout": [ctypes.POINTER(dit_config), ctypes.POINTER(dit_segment), _I, _P, _P, _P, ctypes.POINTER(_I)],
    "dit_rope_cache_build": [ctypes.POINTER(dit_config), ctypes.POINTER(dit_segment), _I, _P, _P],
    "dit_timestep_embedding": [_P, _I, _I, _P],
    "dit_sigma_schedule": [ctypes.c_double, _I, _P, _P],
    "dit_weight_bytes": [ctypes.POINTER(dit_config), ctypes.POINTER(_SZ)],
    "dit_model_create": [ctypes.POINTER(dit_config), _P, _SZ, ctypes.POINTER(_P)],
    "dit_stage_weights": [_P, ctypes.POINTER(dit_weight_view), _I, _P],
    "dit_stage_finalize": [_P],
    "dit_stage_stats": [_P, ctypes.POINTER(dit_stage_stats_t)],
    "dit_batch_bytes": [_P, ctypes.POINTER(dit_segment), _I, ctypes.POINTER(_SZ)],
    "dit_batch_create": [_P, ctypes.POINTER(dit_segment), _I, _I, ctypes.POINTER(_I), _P, _SZ, _P, ctypes.POINTER(_P)],
    "dit_batch_info": [_P, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(ctypes.c_int64)],
    "dit_batch_tables": [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P)],
    "dit_workspace_bytes": [_P, _P, ctypes.POINTER(_SZ)],
    "dit_modulation": [_P, _P, _I, _I, _P, _P, _P],
    "dit_block_forward": [_P, _I, _P, _P, _P, _P, _SZ, _P],
    "dit_forward": [_P, _P, _P, _P, _P, _P, _SZ, _P],
    "dit_denoise_step": [_P, _P, _P, _P, _P, _P, _SZ, _P],
    "dit_denoise_loop": [_P, _P, _P, _P, _P, _I, _P, _SZ, _P],
    "dit_cfg_denoise_loop": [_P, _P, _P, _P, _P, ctypes.c_float, _I, _P, _SZ, _P],
    "dit_gemm_workspace_bytes": [_I, _I, _I, _I, ctypes.POINTER(_SZ)],
    "dit_gemm_splits": [_I, _I, _I, ctypes.POINTER(_I)],
    "dit_gemm_split_groups": [_I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I)],
    "dit_gemm": [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _SZ, _P],
    "dit_gemm_f32_noalloc": [_I, _I, _I, _P, _P, _P, _P, _P],
    "dit_quantize_mx8": [_I, _I, _P, _P, _P, _P],
    "dit_quantize_mx4": [_I, _I, _P, _P, _P, _P],
    "dit_modnorm": [_I, _I, ctypes.c_float, _I, _I, _P, _I, _P, _I, _P, _P, _P],
    "dit_rope_split": [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P],
    "dit_attention": [_I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P],
    "dit_silu_gate": [_I, _I, _I, _P, _P, _P],
    "dit_gated_residual": [_I, _I, _P, _I, _P, _P, _I, _P, _P],
    "dit_counters": [ctypes.POINTER(ctypes.c_int64), _I],
    "dit_profile_begin": [],
    "dit_profile_end": [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double), _I],
    "dit_forward_graph_create": [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p)],
    "dit_graph_launch": [_P, _P],
    "dit_graph_nodes": [_P, ctypes.POINTER(ctypes.c_size_t)],
}
_VOID = {"dit_model_destroy": [_P], "dit_batch_destroy": [_P], "dit_counters_reset": [],
         "dit_graph_destroy": [_P]}

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libdit.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m video_audio_gen_amd.build`")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    for name, args in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    for name, args in _VOID.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = None
    lib.dit_last_error.argtypes = []
    lib.dit_last_error.restype = ctypes.c_char_p
    lib.dit_gemm_f32_noalloc_limit.argtypes = []
    lib.dit_gemm_f32_noalloc_limit.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _check(code: int):
    if code != DIT_OK:
        raise DitError(code, load().dit_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ----------------------------------------------------------------------------- config marshalling

def make_config(spec) -> dit_config:
    """A dit_config from any object with the model-shape attributes (duck-typed)."""
    c = dit_config()
    c.n_blocks, c.hidden, c.n_heads, c.head_dim, c.ffn = (spec.n_blocks, spec.hidden, spec.n_heads,
                                                          spec.head_dim, spec.ffn)
    c.norm = DIT_NORM_RMS if spec.norm == "rms" else DIT_NORM_LAYER
    c.norm_eps = spec.norm_eps
    c.mlp = DIT_MLP_GATE_UP if spec.mlp == "gate_up" else DIT_MLP_VALUE_GATE
    c.rot_dim = spec.rot_dim
    c.theta = spec.theta
    c.stream_dtype = DIT_BF16 if spec.stream == "bf16" else DIT_F32
    c.cond_dim = spec.cond_dim
    c.n_mod = len(spec.modalities)
    c.io = 1 if spec.io else 0
    c.gemm_format = {"mxfp8": DIT_GEMM_MXFP8, "mxfp4": DIT_GEMM_MXFP4}.get(getattr(spec, "gemm", "stream"), DIT_GEMM_STREAM)
    c.qkv_layout = 1 if getattr(spec, "qkv_layout", "concat") == "per_head" else 0
    c.qk_norm = 1 if getattr(spec, "qk_norm", False) else 0
    for i, m in enumerate(spec.modalities):
        md = c.mod[i]
        md.io = {"none": DIT_IO_NONE, "patch3d": DIT_IO_PATCH3D, "channel_major": DIT_IO_CHANNEL_MAJOR}[m.io]
        md.channels = m.channels
        for a in range(3):
            md.patch[a] = m.patch[a]
        md.n_axes = len(m.rope_axes)
        md.rope_grid = 1 if getattr(m, "rope_grid", "integer") == "centered" else 0
        for a in range(md.n_axes):
            md.axis_dim[a] = m.rope_axes[a]
    return c


def make_segments(segments) -> ctypes.Array:
    arr = (dit_segment * len(segments))()
    for i, s in enumerate(segments):
        arr[i].modality = s.modality
        arr[i].cond_row = s.cond_row
        g = list(s.grid) + [1] * (3 - len(s.grid))
        for a in range(3):
            arr[i].grid[a] = g[a]
    return arr


# ----------------------------------------------------------------------------- host builders

def dit_pack_layout(spec, segments=None):
    lib = load()
    cfg = make_config(spec)
    segs = make_segments(segments if segments is not None else spec.segments)
    n = ctypes.c_int()
    cu = np.zeros(len(segs) + 1, np.int32)
    _check(lib.dit_pack_layout(ctypes.byref(cfg), segs, len(segs), cu.ctypes.data, None, None, ctypes.byref(n)))
    ci = np.zeros(n.value, np.int32)
    doc = np.zeros(n.value, np.int32)
    _check(lib.dit_pack_layout(ctypes.byref(cfg), segs, len(segs), cu.ctypes.data, ci.ctypes.data, doc.ctypes.data,
                               ctypes.byref(n)))
    return {"cu_seqlens": cu, "cond_idx": ci, "doc_id": doc}


def dit_rope_cache_build(spec, segments=None):
    lib = load()
    cfg = make_config(spec)
    segs = make_segments(segments if segments is not None else spec.segments)
    N = int(dit_pack_layout(spec, segments)["cu_seqlens"][-1])
    half = spec.rot_dim // 2
    cos = np.zeros((N, half), np.float32)
    sin = np.zeros((N, half), np.float32)
    _check(lib.dit_rope_cache_build(ctypes.byref(cfg), segs, len(segs), cos.ctypes.data, sin.ctypes.data))
    return cos, sin


def dit_timestep_embedding(t: Sequence[float], dim: int) -> np.ndarray:
    t = np.ascontiguousarray(np.asarray(t, np.float32).reshape(-1))
    out = np.zeros((t.size, dim), np.float32)
    _check(load().dit_timestep_embedding(t.ctypes.data, t.size, dim, out.ctypes.data))
    return out


def dit_sigma_schedule(shift: float, n_steps: int):
    sig = np.zeros(n_steps + 1, np.float64)
    dt = np.zeros(n_steps, np.float32)
    _check(load().dit_sigma_schedule(float(shift), n_steps, sig.ctypes.data, dt.ctypes.data))
    return sig, dt


# ----------------------------------------------------------------------------- model

class Model:
    """dit_model plus the torch-allocated weight slab it is bound to."""

    def __init__(self, spec, device="cuda"):
        lib = load()
        self.spec = spec
        self.cfg = make_config(spec)
        nbytes = ctypes.c_size_t()
        _check(lib.dit_weight_bytes(ctypes.byref(self.cfg), ctypes.byref(nbytes)))
        self.slab = torch.empty(max(int(nbytes.value), 256) + 256, dtype=torch.uint8, device=device)
        base = self.slab.data_ptr()
        aligned = (base + 255) & ~255
        h = ctypes.c_void_p()
        _check(lib.dit_model_create(ctypes.byref(self.cfg), aligned, int(nbytes.value), ctypes.byref(h)))
        self.handle = h
        self.weight_bytes = int(nbytes.value)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            load().dit_model_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _bf16_exact(a: np.ndarray) -> bool:
    return not (a.reshape(-1).view(np.uint32) & np.uint32(0xFFFF)).any()


def dit_stage_weights(model: Model, tensors: Dict[str, np.ndarray], stream=None, as_bf16: bool = False):
    """Stage host arrays by name.  float32 arrays are sent as f32 views (the
    library rounds them for a bf16 stream).  With ``as_bf16``, a float32 array
    whose values are all bf16-representable is sent as its raw bf16 bits
    instead (half the host-to-device bytes); any other array is sent as is."""
    keep = []
    views = (dit_weight_view * len(tensors))()
    for i, (name, a) in enumerate(tensors.items()):
        a = np.ascontiguousarray(a)
        if as_bf16 and a.dtype == np.float32 and a.ndim == 2 and _bf16_exact(a):
            a = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        if a.dtype == np.uint16:
            dt = DIT_BF16
        elif a.dtype == np.float32:
            dt = DIT_F32
        else:
            raise TypeError(f"{name}: dtype {a.dtype}")
        keep.append(a)
        nb = name.encode()
        keep.append(nb)
        views[i].name = nb
        views[i].dtype = dt
        views[i].ndim = a.ndim
        for d in range(a.ndim):
            views[i].shape[d] = a.shape[d]
        views[i].host = a.ctypes.data
    _check(load().dit_stage_weights(model.handle, views, len(tensors), _stream(stream)))


def dit_stage_finalize(model: Model):
    _check(load().dit_stage_finalize(model.handle))


def dit_stage_stats(model: Model) -> Dict[str, int]:
    s = dit_stage_stats_t()
    _check(load().dit_stage_stats(model.handle, ctypes.byref(s)))
    return {k: getattr(s, k) for k, _ in s._fields_}


# ----------------------------------------------------------------------------- batch

class Batch:
    """dit_batch plus its torch-allocated device tables."""

    def __init__(self, model: Model, segments, cond_modality: Sequence[int], stream=None):
        lib = load()
        self.model = model
        self.segs = make_segments(segments)
        nbytes = ctypes.c_size_t()
        _check(lib.dit_batch_bytes(model.handle, self.segs, len(self.segs), ctypes.byref(nbytes)))
        self.tables = torch.empty(int(nbytes.value) + 256, dtype=torch.uint8, device=model.slab.device)
        aligned = (self.tables.data_ptr() + 255) & ~255
        cm = (ctypes.c_int * len(cond_modality))(*cond_modality)
        h = ctypes.c_void_p()
        _check(lib.dit_batch_create(model.handle, self.segs, len(self.segs), len(cond_modality), cm, aligned,
                                    int(nbytes.value), _stream(stream), ctypes.byref(h)))
        self.handle = h
        self.n_cond = len(cond_modality)
        n, ns, ms = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        lf = ctypes.c_int64()
        _check(lib.dit_batch_info(h, ctypes.byref(n), ctypes.byref(ns), ctypes.byref(ms), ctypes.byref(lf)))
        self.n_tokens, self.n_segs, self.max_seqlen, self.latent_floats = n.value, ns.value, ms.value, lf.value
        ws = ctypes.c_size_t()
        _check(lib.dit_workspace_bytes(model.handle, h, ctypes.byref(ws)))
        self.workspace_bytes = int(ws.value)

    def tables_ptrs(self):
        p = [ctypes.c_void_p() for _ in range(4)]
        _check(load().dit_batch_tables(self.handle, *[ctypes.byref(x) for x in p]))
        return [x.value for x in p]

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            load().dit_batch_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def workspace(batch: Batch) -> torch.Tensor:
    return torch.empty(max(batch.workspace_bytes, 1), dtype=torch.uint8, device=batch.model.slab.device)


# ----------------------------------------------------------------------------- forward calls

def dit_modulation(model: Model, batch: Batch, block0: int, n_blocks: int, cond, mod, stream=None):
    _check(load().dit_modulation(model.handle, batch.handle, block0, n_blocks, _ptr(cond), _ptr(mod), _stream(stream)))


def dit_block_forward(model: Model, block: int, x, mod, batch: Batch, ws, stream=None):
    _check(load().dit_block_forward(model.handle, block, _ptr(x), _ptr(mod), batch.handle, _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def dit_forward(model: Model, batch: Batch, inp, cond, out, ws, stream=None):
    _check(load().dit_forward(model.handle, batch.handle, _ptr(inp), _ptr(cond), _ptr(out), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)))


class ForwardGraph:
    """dit_forward captured once as a HIP graph (dit_forward_graph_create); launch() replays it.

    Keeps the tensors it was captured on alive: a replay reads their current contents."""

    def __init__(self, model: Model, batch: Batch, inp, cond, out, ws):
        self._keep = (model, batch, inp, cond, out, ws)
        h = ctypes.c_void_p()
        _check(load().dit_forward_graph_create(model.handle, batch.handle, _ptr(inp), _ptr(cond), _ptr(out), _ptr(ws),
                                               ws.numel() * ws.element_size(), ctypes.byref(h)))
        self.handle = h

    def launch(self, stream=None):
        _check(load().dit_graph_launch(self.handle, _stream(stream)))

    @property
    def nodes(self) -> int:
        n = ctypes.c_size_t()
        _check(load().dit_graph_nodes(self.handle, ctypes.byref(n)))
        return int(n.value)

    def close(self):
        if self.handle is not None and self.handle.value is not None:
            load().dit_graph_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dit_denoise_step(model: Model, batch: Batch, latents, cond, dt, ws, stream=None):
    _check(load().dit_denoise_step(model.handle, batch.handle, _ptr(latents), _ptr(cond), _ptr(dt), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def dit_denoise_loop(model: Model, batch: Batch, latents, cond_table, dt_table, n_steps: int, ws, stream=None):
    _check(load().dit_denoise_loop(model.handle, batch.handle, _ptr(latents), _ptr(cond_table), _ptr(dt_table),
                                   n_steps, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dit_cfg_denoise_loop(model: Model, batch: Batch, latents, cond_table, dt_table, w: float, n_steps: int, ws,
                         stream=None):
    _check(load().dit_cfg_denoise_loop(model.handle, batch.handle, _ptr(latents), _ptr(cond_table), _ptr(dt_table),
                                       float(w), n_steps, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


# ----------------------------------------------------------------------------- op-level calls

def _dt(t) -> int:
    if t.dtype in (torch.float32,):
        return DIT_F32
    if t.dtype == torch.float64:
        return DIT_F64
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DIT_BF16
    raise TypeError(t.dtype)


def dit_quantize_mx8(x, codes, scales, stream=None):
    """bf16 rows x [R, K] -> E4M3 codes [R, K] (uint8) and E8M0 scales [R, K/32] (uint8)."""
    R, K = x.shape
    _check(load().dit_quantize_mx8(R, K, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))


def dit_quantize_mx4(x, codes, scales, stream=None):
    """bf16 rows x [R, K] -> E2M1 codes [R, K/2] (uint8, two per byte) and E8M0 scales [R, K/32] (uint8)."""
    R, K = x.shape
    _check(load().dit_quantize_mx4(R, K, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))


def dit_gemm(A, B, bias, C, stream=None, mxfp8=False, mxfp4=False):
    """C[M,N] = A[M,K] . B[N,K]^T + bias (mxfp8: bf16 A, B re-quantized to MXFP8 first;
    mxfp4: A to MXFP8 and B to MXFP4)."""
    M, K = A.shape
    N = B.shape[0]
    dt = DIT_MXFP4 if mxfp4 else DIT_MXFP8 if mxfp8 else _dt(A)
    ws_bytes = ctypes.c_size_t()
    _check(load().dit_gemm_workspace_bytes(dt, M, N, K, ctypes.byref(ws_bytes)))
    ws = torch.empty(max(int(ws_bytes.value), 1), dtype=torch.uint8, device=A.device)
    _check(load().dit_gemm(dt, M, N, K, _ptr(A), _ptr(B), _ptr(bias), _ptr(C), _dt(C), _ptr(ws), int(ws_bytes.value),
                           _stream(stream)))
    return ws


def dit_gemm_f32_noalloc(A, B, bias, C, stream=None):
    """fp32 C[M,N] = A[M,K] . B[N,K]^T + bias with the library's built-in scratch (no workspace)."""
    M, K = A.shape
    N = B.shape[0]
    _check(load().dit_gemm_f32_noalloc(M, N, K, _ptr(A), _ptr(B), _ptr(bias), _ptr(C), _stream(stream)))


def dit_gemm_f32_noalloc_limit() -> int:
    return int(load().dit_gemm_f32_noalloc_limit())


def dit_gemm_splits(N: int, K: int) -> int:
    """Split-K count of the fp32 GEMM for an [N, K] weight on the current device."""
    s = ctypes.c_int()
    _check(load().dit_gemm_splits(DIT_F32, N, K, ctypes.byref(s)))
    return int(s.value)


def dit_gemm_split_groups(N: int, K: int):
    """(s_lo, s_hi, col_split) of the fp32 GEMM for an [N, K] weight on the current device."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load().dit_gemm_split_groups(DIT_F32, N, K, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return int(a.value), int(b.value), int(c.value)


def dit_modnorm(norm: int, eps: float, x, mod, which: int, cond_idx, h, stream=None):
    N, D = x.shape
    _check(load().dit_modnorm(_dt(h), norm, eps, N, D, _ptr(x), _dt(x), _ptr(mod), which, _ptr(cond_idx), _ptr(h),
                              _stream(stream)))


def dit_rope_split(qkv, H: int, hd: int, rot: int, cos, sin, q, k, v, stream=None):
    N = qkv.shape[0]
    _check(load().dit_rope_split(_dt(qkv), N, H, hd, rot, _ptr(qkv), _ptr(cos), _ptr(sin), _ptr(q), _ptr(k), _ptr(v),
                                 _stream(stream)))


def dit_attention(q, k, v, cu_seqlens, max_seqlen: int, o, stream=None):
    H, N, hd = q.shape
    _check(load().dit_attention(_dt(q), N, H, hd, cu_seqlens.numel() - 1, _ptr(cu_seqlens), max_seqlen, _ptr(q),
                                _ptr(k), _ptr(v), _ptr(o), _stream(stream)))


def dit_silu_gate(u, m, stream=None):
    N, F2 = u.shape
    _check(load().dit_silu_gate(_dt(u), N, F2 // 2, _ptr(u), _ptr(m), _stream(stream)))


def dit_gated_residual(x, a, mod, which: int, cond_idx, stream=None):
    N, D = x.shape
    _check(load().dit_gated_residual(N, D, _ptr(x), _dt(x), _ptr(a), _ptr(mod), which, _ptr(cond_idx),
                                     _stream(stream)))


def dit_counters() -> Dict[str, int]:
    arr = (ctypes.c_int64 * len(COUNTER_NAMES))()
    _check(load().dit_counters(arr, len(COUNTER_NAMES)))
    return dict(zip(COUNTER_NAMES, list(arr)))


def dit_counters_reset():
    load().dit_counters_reset()


def dit_profile_begin():
    _check(load().dit_profile_begin())


def dit_profile_end() -> Dict[str, Tuple[int, float]]:
    """{kernel family: (launches, summed device ms)} since dit_profile_begin."""
    n = len(COUNTER_NAMES)
    cnt = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    _check(load().dit_profile_end(cnt, ms, n))
    return {name: (int(cnt[i]), float(ms[i])) for i, name in enumerate(COUNTER_NAMES)}
