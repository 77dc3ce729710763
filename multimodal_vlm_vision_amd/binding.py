"""ctypes binding of include/vit.h (argument marshalling only).

Every step of the forward runs inside libvitmi.so; this module only converts
Python/NumPy/torch arguments into the C ABI's plain pointers and sizes.
torch is used for device memory and streams.  Importing this module fails
loudly if the library has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libvitmi.so")
HEADER = os.path.join(ROOT, "include", "vit.h")

VIT_OK, VIT_E_ARG, VIT_E_SHAPE, VIT_E_WEIGHTS, VIT_E_WORKSPACE, VIT_E_STATE, VIT_E_HIP = range(7)
VIT_MLP_GELU, VIT_MLP_SWIGLU = 0, 1
VIT_NORM_LAYER, VIT_NORM_RMS = 0, 1
VIT_F32, VIT_BF16 = 0, 1
VIT_ACT_BF16, VIT_ACT_BF16X2, VIT_ACT_BF16F8, VIT_ACT_F16 = 0, 1, 2, 3
MAX_FULL_LAYERS = 64

_STATUS_NAMES = {0: "VIT_OK", 1: "VIT_E_ARG", 2: "VIT_E_SHAPE", 3: "VIT_E_WEIGHTS",
                 4: "VIT_E_WORKSPACE", 5: "VIT_E_STATE", 6: "VIT_E_HIP"}


class VitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class vit_config(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32), ("layers", ctypes.c_int32),
        ("mlp_dim", ctypes.c_int32), ("mlp_kind", ctypes.c_int32), ("norm_kind", ctypes.c_int32),
        ("norm_eps", ctypes.c_float), ("patch", ctypes.c_int32), ("temporal_patch", ctypes.c_int32),
        ("merge", ctypes.c_int32), ("out_dim", ctypes.c_int32), ("rope_theta", ctypes.c_float),
        ("mean", ctypes.c_float * 3), ("std", ctypes.c_float * 3), ("window_px", ctypes.c_int32),
        ("n_full_attn_layers", ctypes.c_int32), ("full_attn_layers", ctypes.c_int32 * MAX_FULL_LAYERS),
        ("activation_precision", ctypes.c_int32),
    ]


class vit_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("mfma_bound", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


_P = ctypes.c_void_p
_SIGS = {
    "vit_last_error": (ctypes.c_char_p, []),
    "vit_create": (ctypes.c_int32, [ctypes.POINTER(vit_config), ctypes.POINTER(_P)]),
    "vit_load_weight": (ctypes.c_int32, [_P, ctypes.c_char_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int32, _P]),
    "vit_finalize_weights": (ctypes.c_int32, [_P, _P]),
    "vit_plan_create": (ctypes.c_int32, [_P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                         ctypes.c_int32, ctypes.POINTER(_P)]),
    "vit_plan_destroy": (None, [_P]),
    "vit_plan_sizes": (ctypes.c_int32, [_P, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    "vit_plan_rows": (ctypes.c_int32, [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]),
    "vit_plan_attention_units": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                                  ctypes.POINTER(ctypes.c_int32)]),
    "vit_encode": (ctypes.c_int32, [_P, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "vit_encode_patches_u8": (ctypes.c_int32, [_P, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "vit_encode_noalloc": (ctypes.c_int32, [_P, _P, _P, _P, _P]),
    "vit_graph_capture": (ctypes.c_int32, [_P, _P, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]),
    "vit_graph_io": (ctypes.c_int32, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P)]),
    "vit_graph_launch": (ctypes.c_int32, [_P, _P]),
    "vit_graph_capture_bucket": (ctypes.c_int32, [_P, _P, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]),
    "vit_graph_launch_plan": (ctypes.c_int32, [_P, _P, _P]),
    "vit_cache_create": (ctypes.c_int32, [_P, _P, ctypes.c_size_t, ctypes.POINTER(_P)]),
    "vit_cache_stats": (ctypes.c_int32, [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)]),
    "vit_cache_destroy": (None, [_P]),
    "vit_encode_cached": (ctypes.c_int32, [_P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P,
                                           ctypes.POINTER(ctypes.c_int32)]),
    "vit_pixel_keys": (ctypes.c_int32, [_P, _P, _P, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint64), _P]),
    "vit_resize_side": (ctypes.c_int32, [ctypes.c_int32]),
    "vit_resize_u8": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t, _P]),
    "vit_graph_destroy": (None, [_P]),
    "vit_destroy": (None, [_P]),
    "vit_encode_profiled": (ctypes.c_int32, [_P, _P, _P, _P, ctypes.c_size_t, _P, _P,
                                             ctypes.POINTER(vit_kernel_stat), ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int32)]),
    "vit_debug_stage": (ctypes.c_int32, [_P, _P, _P, _P, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, _P,
                                         ctypes.c_size_t, _P]),
}

_lib: Optional[ctypes.CDLL] = None


def header_symbols() -> list:
    """Names of the functions include/vit.h declares."""
    text = open(HEADER).read()
    decl = r"^\s*(?:const\s+char\s*\*|vit_status|void|int32_t)\s+(vit_[a-z_0-9]+)\s*\("
    return sorted(set(re.findall(decl, text, flags=re.M)))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built (python -m multimodal_vlm_vision_amd.build); "
                          "the vision tower has no other implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(lib, status: int):
    if status != VIT_OK:
        raise VitError(status, lib.vit_last_error().decode())


def make_config(cfg, activation_precision: str = "f16") -> vit_config:
    """vit_config from any object with the tower fields (e.g. workloads.TowerConfig).

    activation_precision: "f16" (every GEMM and attention activation in float16 against
    float16 weight copies; the default), "bf16f8" (the norm, attention-output, MLP and
    merger GEMM inputs as bf16 plus an e4m3 residual), "bf16x2" (the same activations as
    hi+lo bf16 pairs) or "bf16" (rounded once)."""
    c = vit_config()
    c.activation_precision = {"bf16": VIT_ACT_BF16, "bf16x2": VIT_ACT_BF16X2,
                              "bf16f8": VIT_ACT_BF16F8, "f16": VIT_ACT_F16}[activation_precision]
    c.hidden, c.heads, c.layers, c.mlp_dim = cfg.hidden, cfg.heads, cfg.layers, cfg.mlp_dim
    c.mlp_kind = VIT_MLP_GELU if cfg.mlp_kind == "gelu" else VIT_MLP_SWIGLU
    c.norm_kind = VIT_NORM_LAYER if cfg.norm_kind == "layer" else VIT_NORM_RMS
    c.norm_eps = cfg.norm_eps
    c.patch, c.temporal_patch, c.merge = cfg.patch, cfg.temporal_patch, cfg.merge
    c.out_dim = cfg.out_dim
    c.rope_theta = cfg.rope_theta
    for i in range(3):
        c.mean[i] = cfg.mean[i]
        c.std[i] = cfg.std[i]
    c.window_px = cfg.window_px
    full = list(cfg.full_attn_layers)
    c.n_full_attn_layers = len(full)
    for i, l in enumerate(full):
        c.full_attn_layers[i] = l
    return c


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


class Plan:
    def __init__(self, tower: "VisionTower", grid_thw: np.ndarray, n_frames: np.ndarray):
        self.lib = tower.lib
        g = np.ascontiguousarray(np.asarray(grid_thw, dtype=np.int32).reshape(-1, 3))
        f = np.ascontiguousarray(np.asarray(n_frames, dtype=np.int32).reshape(-1))
        self.handle = _P()
        self.n_items = len(f)
        _check(self.lib, self.lib.vit_plan_create(
            tower.handle, g.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            f.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(f), ctypes.byref(self.handle)))
        px, ws = ctypes.c_size_t(), ctypes.c_size_t()
        rows, cols = ctypes.c_int64(), ctypes.c_int64()
        _check(self.lib, self.lib.vit_plan_sizes(self.handle, ctypes.byref(px), ctypes.byref(ws),
                                                 ctypes.byref(rows), ctypes.byref(cols)))
        self.pixel_bytes, self.ws_bytes = px.value, ws.value
        self.out_rows, self.out_cols = rows.value, cols.value
        n = ctypes.c_int64()
        _check(self.lib, self.lib.vit_plan_rows(self.handle, ctypes.byref(n), None))
        self.n_patches = n.value

    def row_order(self) -> np.ndarray:
        out = np.zeros(self.n_patches, dtype=np.int32)
        n = ctypes.c_int64()
        _check(self.lib, self.lib.vit_plan_rows(self.handle, ctypes.byref(n),
                                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return out

    def attention_units(self, windows: bool = False, split: bool = True):
        """The long attention work units (rows of: segment start, segment length, first query,
        first and end key block, partial slot or -1, 0, 0), the number of merged query blocks
        and of partial slots; split=False gives the plain list."""
        n, nm, npart = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self.lib, self.lib.vit_plan_attention_units(self.handle, int(windows), int(split), None,
                                                           ctypes.byref(n), ctypes.byref(nm), ctypes.byref(npart)))
        out = np.zeros((n.value, 8), dtype=np.int32)
        _check(self.lib, self.lib.vit_plan_attention_units(self.handle, int(windows), int(split),
                                                           out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                           ctypes.byref(n), ctypes.byref(nm), ctypes.byref(npart)))
        return out, nm.value, npart.value

    def close(self):
        if self.handle:
            self.lib.vit_plan_destroy(self.handle)
            self.handle = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Graph:
    """vit_graph_capture, or vit_graph_capture_bucket when bucket=True (plan = the capacity)."""

    def __init__(self, tower, plan: Plan, ws, stream=None, bucket: bool = False):
        self.lib = tower.lib
        self.handle = _P()
        self._keep = (tower, plan, ws)
        capture = self.lib.vit_graph_capture_bucket if bucket else self.lib.vit_graph_capture
        _check(self.lib, capture(tower.handle, plan.handle, _ptr(ws), ws.numel(),
                                 _stream_handle(stream), ctypes.byref(self.handle)))
        pin, pout = _P(), _P()
        _check(self.lib, self.lib.vit_graph_io(self.handle, ctypes.byref(pin), ctypes.byref(pout)))
        self.pixels_ptr, self.out_ptr = pin.value, pout.value

    def launch(self, stream=None):
        _check(self.lib, self.lib.vit_graph_launch(self.handle, _stream_handle(stream)))

    def launch_plan(self, plan: Plan, stream=None):
        """Bucketed graph: replay for another plan that fits the captured capacity."""
        _check(self.lib, self.lib.vit_graph_launch_plan(self.handle, plan.handle, _stream_handle(stream)))

    def close(self):
        if self.handle:
            self.lib.vit_graph_destroy(self.handle)
            self.handle = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def resize_side(pixels: int, lib: Optional[ctypes.CDLL] = None) -> int:
    """vit_resize_side: the 28-multiple a side of `pixels` resizes to."""
    return int((lib or load_library()).vit_resize_side(int(pixels)))


def resize_u8(src, sh: int, sw: int, frames: int, dst, stream=None, lib: Optional[ctypes.CDLL] = None):
    """vit_resize_u8 on device uint8 tensors (frames x sh x sw x 3 -> frames x dh x dw x 3)."""
    lib = lib or load_library()
    _check(lib, lib.vit_resize_u8(_ptr(src), sh, sw, frames, _ptr(dst), dst.numel(), _stream_handle(stream)))


class EmbeddingCache:
    """vit_cache over a caller-owned device arena (a uint8 torch tensor)."""

    def __init__(self, tower, arena):
        self.lib = tower.lib
        self.handle = _P()
        self._keep = (tower, arena)
        n = arena.numel() if arena is not None else 0
        _check(self.lib, self.lib.vit_cache_create(tower.handle, _ptr(arena), n, ctypes.byref(self.handle)))

    def stats(self):
        e, b = ctypes.c_int64(), ctypes.c_size_t()
        _check(self.lib, self.lib.vit_cache_stats(self.handle, ctypes.byref(e), ctypes.byref(b)))
        return e.value, b.value

    def close(self):
        if self.handle:
            self.lib.vit_cache_destroy(self.handle)
            self.handle = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class VisionTower:
    """Owns one vit_ctx: configuration, weights (host copies until finalize, then a device arena)."""

    def __init__(self, cfg, lib: Optional[ctypes.CDLL] = None, activation_precision: str = "f16"):
        self.lib = lib or load_library()
        self.cfg = cfg
        self.activation_precision = activation_precision
        # debug stages of the compensated activations come as [hi | lo] rows in both forms
        self.split = 2 if activation_precision in ("bf16x2", "bf16f8") else 1
        c = make_config(cfg, activation_precision)
        self.handle = _P()
        _check(self.lib, self.lib.vit_create(ctypes.byref(c), ctypes.byref(self.handle)))

    def load_weight(self, name: str, array: np.ndarray, dtype: int = VIT_F32):
        a = np.ascontiguousarray(array, dtype=np.float32 if dtype == VIT_F32 else np.uint16)
        shape = (ctypes.c_int64 * a.ndim)(*a.shape)
        _check(self.lib, self.lib.vit_load_weight(self.handle, name.encode(), dtype, shape, a.ndim,
                                                  a.ctypes.data_as(_P)))

    def load_weights(self, weights: Dict[str, np.ndarray]):
        for name, arr in weights.items():
            self.load_weight(name, arr)

    def finalize(self, stream=None):
        _check(self.lib, self.lib.vit_finalize_weights(self.handle, _stream_handle(stream)))

    def plan(self, grid_thw, n_frames) -> Plan:
        return Plan(self, grid_thw, n_frames)

    def encode(self, plan: Plan, pixels, ws, out, stream=None):
        _check(self.lib, self.lib.vit_encode(self.handle, plan.handle, _ptr(pixels), _ptr(ws),
                                             ws.numel() if ws is not None else 0, _ptr(out),
                                             _stream_handle(stream)))

    def encode_noalloc(self, plan: Plan, pixels, out, stream=None):
        """vit_encode with the library's static device scratch as the workspace (no allocation)."""
        _check(self.lib, self.lib.vit_encode_noalloc(self.handle, plan.handle, _ptr(pixels), _ptr(out),
                                                     _stream_handle(stream)))

    def encode_patches_u8(self, plan: Plan, patches, ws, out, stream=None):
        _check(self.lib, self.lib.vit_encode_patches_u8(self.handle, plan.handle, _ptr(patches), _ptr(ws),
                                                        ws.numel(), _ptr(out), _stream_handle(stream)))

    def encode_profiled(self, plan: Plan, pixels, ws, out, stream=None) -> list:
        """Forward with per-launch hipEvents; returns [{name, launches, total_ms, flops, bytes, mfma_bound}]."""
        stats = (vit_kernel_stat * 64)()
        n = ctypes.c_int32()
        _check(self.lib, self.lib.vit_encode_profiled(self.handle, plan.handle, _ptr(pixels), _ptr(ws), ws.numel(),
                                                      _ptr(out), _stream_handle(stream), stats, 64, ctypes.byref(n)))
        return [{"name": stats[i].name.decode(), "launches": stats[i].launches, "total_ms": stats[i].total_ms,
                 "flops": stats[i].flops, "bytes": stats[i].bytes, "mfma_bound": bool(stats[i].mfma_bound)}
                for i in range(min(n.value, 64))]

    def debug_stage(self, plan: Plan, pixels, ws, layer: int, step: int, dst, stream=None):
        _check(self.lib, self.lib.vit_debug_stage(self.handle, plan.handle, _ptr(pixels), _ptr(ws), ws.numel(),
                                                  layer, step, _ptr(dst), dst.numel() * dst.element_size(),
                                                  _stream_handle(stream)))

    def capture(self, plan: Plan, ws, stream=None) -> Graph:
        return Graph(self, plan, ws, stream)

    def encode_cached(self, cache: "EmbeddingCache", plan: Plan, pixels, ws, out, stream=None) -> int:
        """vit_encode through the embedding cache; returns the number of items served from it."""
        hits = ctypes.c_int32()
        _check(self.lib, self.lib.vit_encode_cached(self.handle, cache.handle, plan.handle, _ptr(pixels), _ptr(ws),
                                                    ws.numel() if ws is not None else 0, _ptr(out),
                                                    _stream_handle(stream), ctypes.byref(hits)))
        return hits.value

    def pixel_keys(self, plan: Plan, pixels, ws, stream=None) -> np.ndarray:
        """[n_items][2] uint64 content keys of the items' pixels."""
        keys = np.zeros((plan.n_items, 2), dtype=np.uint64)
        _check(self.lib, self.lib.vit_pixel_keys(self.handle, plan.handle, _ptr(pixels), _ptr(ws),
                                                 ws.numel() if ws is not None else 0,
                                                 keys.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                                 _stream_handle(stream)))
        return keys

    def capture_bucket(self, plan: Plan, ws, stream=None) -> Graph:
        """Bucketed graph for the capacity `plan`; replay other plans with Graph.launch_plan."""
        return Graph(self, plan, ws, stream, bucket=True)

    def close(self):
        if self.handle:
            self.lib.vit_destroy(self.handle)
            self.handle = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
