"""The five tower workloads and their seeded input recipe.

Tower shapes follow the Qwen2-VL / Qwen2.5-VL vision tower as the pages
describe it: 14-pixel patches, temporal patch 2, 2x2 spatial merge, a
(c, tau, i, j)-ordered flattened patch of 3*2*14*14 = 1176 features, 2D
rotary positions and a patch-merger MLP (vLLM multimodal ViT optimisation
blog, sections 2.2 and 3.2-3.3).  Sizes, layer counts and the per-workload
choices (LayerNorm/GELU vs RMSNorm/SwiGLU, 112 px windows) are the workload
definitions themselves.

Draw recipe (every stream is an independent ``numpy.random.PCG64`` keyed by
a ``SeedSequence``):

* item sizes:      SeedSequence([cfg, 0])          (one stream, redrawn as a set)
* pixels of item i SeedSequence([cfg, 1, i])       uniform uint8 in [0, 255]
* block weight     SeedSequence([cfg, 2, layer, slot])
* other weights    SeedSequence([cfg, 3, slot])

Matrices and biases are N(0, 0.02); norm gains are 1 + N(0, 0.02) and norm
shifts N(0, 0.02).  For bf16-weight workloads each draw is rounded to the
nearest bfloat16 (ties to even) *here*, so the oracle and the library
receive identical, exactly representable values.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

CONFIG_IDS = (1, 2, 3, 4, 5)

PATCH = 14
TEMPORAL_PATCH = 2
MERGE = 2


@dataclasses.dataclass(frozen=True)
class TowerConfig:
    name: str
    hidden: int
    heads: int
    layers: int
    mlp_dim: int
    mlp_kind: str            # "gelu" (fc1 -> GELU -> fc2) or "swiglu" (gate/up -> SiLU*mul -> down)
    norm_kind: str           # "layer" or "rms"
    out_dim: int
    window_px: int = 0       # 0: no window attention
    full_attn_layers: Tuple[int, ...] = ()
    weight_dtype: str = "bf16"   # "f32" or "bf16"
    patch: int = PATCH
    temporal_patch: int = TEMPORAL_PATCH
    merge: int = MERGE
    norm_eps: float = 1e-6
    rope_theta: float = 10000.0
    mean: Tuple[float, float, float] = (0.48, 0.46, 0.41)
    std: Tuple[float, float, float] = (0.27, 0.26, 0.28)

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def patch_features(self) -> int:
        return 3 * self.temporal_patch * self.patch * self.patch

    @property
    def merge_dim(self) -> int:
        return self.hidden * self.merge * self.merge

    def with_layers(self, layers: int) -> "TowerConfig":
        full = tuple(l for l in self.full_attn_layers if l < layers)
        return dataclasses.replace(self, layers=layers, full_attn_layers=full)


@dataclasses.dataclass
class Item:
    frames: np.ndarray       # uint8 [F][H][W][3], HWC RGB
    grid_thw: Tuple[int, int, int]

    @property
    def n_frames(self) -> int:
        return int(self.frames.shape[0])

    @property
    def n_patches(self) -> int:
        t, h, w = self.grid_thw
        return t * h * w


@dataclasses.dataclass
class Workload:
    index: int
    cfg: TowerConfig
    items: List[Item]
    weights: Dict[str, np.ndarray]

    @property
    def grid_thw(self) -> np.ndarray:
        return np.array([it.grid_thw for it in self.items], dtype=np.int32).reshape(-1, 3)

    @property
    def n_frames(self) -> np.ndarray:
        return np.array([it.n_frames for it in self.items], dtype=np.int32)

    @property
    def n_patches(self) -> int:
        return sum(it.n_patches for it in self.items)

    @property
    def seg_lengths(self) -> List[int]:
        return [it.n_patches for it in self.items]


def tower_config(index: int) -> TowerConfig:
    if index == 1:
        return TowerConfig("tiny-1img-56px", hidden=64, heads=2, layers=1, mlp_dim=256,
                           mlp_kind="gelu", norm_kind="layer", out_dim=128, weight_dtype="f32")
    if index == 2:
        return TowerConfig("qwen2vl-448px-4L", hidden=1280, heads=16, layers=4, mlp_dim=5120,
                           mlp_kind="gelu", norm_kind="layer", out_dim=3584)
    if index == 3:
        return TowerConfig("qwen2vl-8img-mixed-32L", hidden=1280, heads=16, layers=32, mlp_dim=5120,
                           mlp_kind="gelu", norm_kind="layer", out_dim=3584)
    if index == 4:
        return TowerConfig("qwen2vl-video-16f-504x896-32L", hidden=1280, heads=16, layers=32,
                           mlp_dim=5120, mlp_kind="gelu", norm_kind="layer", out_dim=3584)
    if index == 5:
        return TowerConfig("qwen25vl-12img-1vid-window-32L", hidden=1280, heads=16, layers=32,
                           mlp_dim=3420, mlp_kind="swiglu", norm_kind="rms", out_dim=3584,
                           window_px=112, full_attn_layers=(7, 15, 23, 31))
    raise ValueError(f"unknown workload index {index}")


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _grid(n_frames: int, height: int, width: int, tp: int = TEMPORAL_PATCH,
          p: int = PATCH) -> Tuple[int, int, int]:
    t = 1 if n_frames == 1 else n_frames // tp
    return (t, height // p, width // p)


def draw_items(index: int) -> List[Tuple[int, int, int]]:
    """Item sizes (n_frames, H, W) in pixels, in item order."""
    if index == 1:
        return [(1, 56, 56)]
    if index == 2:
        return [(1, 448, 448)]
    if index == 3:
        g = _rng(index, 0)
        sides = 28 * g.integers(8, 49, size=(8, 2))
        return [(1, int(h), int(w)) for h, w in sides]
    if index == 4:
        return [(16, 504, 896)]
    if index == 5:
        g = _rng(index, 0)
        while True:
            img = 28 * g.integers(8, 25, size=(12, 2))
            vid = 28 * g.integers(8, 17, size=2)
            sizes = [(1, int(h), int(w)) for h, w in img] + [(8, int(vid[0]), int(vid[1]))]
            n = sum((h // 14) * (w // 14) * (1 if f == 1 else f // 2) for f, h, w in sizes)
            if 15000 <= n <= 17000:
                return sizes
    raise ValueError(f"unknown workload index {index}")


def _pixels(index: int, item: int, n_frames: int, height: int, width: int) -> np.ndarray:
    return _rng(index, 1, item).integers(0, 256, size=(n_frames, height, width, 3), dtype=np.uint8)


def weight_specs(cfg: TowerConfig) -> List[Tuple[str, Tuple[int, ...], str, Tuple[int, ...]]]:
    """Canonical weight list: (name, shape, kind, seed key).

    kind is "mat" / "bias" (N(0, .02)), "gain" (1 + N(0, .02)) or "shift" (N(0, .02)).
    Linear weights are [out, in]; the patch-embed weight is the conv kernel
    [hidden][3][temporal_patch][patch][patch].
    """
    d, f = cfg.hidden, cfg.mlp_dim
    specs = [("pe.w", (d, 3, cfg.temporal_patch, cfg.patch, cfg.patch), "mat", (3, 0))]

    def norm(prefix: str, key):
        out = [(prefix + ".g", (d,), "gain", key + (0,))]
        if cfg.norm_kind == "layer":
            out.append((prefix + ".b", (d,), "shift", key + (1,)))
        return out

    for l in range(cfg.layers):
        k = lambda slot: (2, l, slot)  # noqa: E731
        specs += norm(f"blk{l}.n1", (2, l, 0))
        specs += [(f"blk{l}.qkv.w", (3 * d, d), "mat", k(2)), (f"blk{l}.qkv.b", (3 * d,), "bias", k(3)),
                  (f"blk{l}.proj.w", (d, d), "mat", k(4)), (f"blk{l}.proj.b", (d,), "bias", k(5))]
        specs += norm(f"blk{l}.n2", (2, l, 6))
        if cfg.mlp_kind == "gelu":
            specs += [(f"blk{l}.fc1.w", (f, d), "mat", k(8)), (f"blk{l}.fc1.b", (f,), "bias", k(9)),
                      (f"blk{l}.fc2.w", (d, f), "mat", k(10)), (f"blk{l}.fc2.b", (d,), "bias", k(11))]
        else:
            specs += [(f"blk{l}.gate.w", (f, d), "mat", k(8)), (f"blk{l}.gate.b", (f,), "bias", k(9)),
                      (f"blk{l}.up.w", (f, d), "mat", k(12)), (f"blk{l}.up.b", (f,), "bias", k(13)),
                      (f"blk{l}.down.w", (d, f), "mat", k(10)), (f"blk{l}.down.b", (d,), "bias", k(11))]
    md = cfg.merge_dim
    specs += norm("mrg.nq", (3, 1))
    specs += [("mrg.fc1.w", (md, md), "mat", (3, 3)), ("mrg.fc1.b", (md,), "bias", (3, 4)),
              ("mrg.fc2.w", (cfg.out_dim, md), "mat", (3, 5)), ("mrg.fc2.b", (cfg.out_dim,), "bias", (3, 6))]
    return specs


def bf16_representable(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _draw_weight(index: int, shape, kind: str, key, bf16: bool) -> np.ndarray:
    g = _rng(index, *key)
    w = g.standard_normal(int(np.prod(shape)), dtype=np.float32)
    w *= np.float32(0.02)
    if kind == "gain":
        w += np.float32(1.0)
    if bf16:
        w = bf16_representable(w)
    return w.reshape(shape)


def make_weights(index: int, cfg: TowerConfig, threads: int = 8) -> Dict[str, np.ndarray]:
    specs = weight_specs(cfg)
    bf16 = cfg.weight_dtype == "bf16"

    def one(spec):
        name, shape, kind, key = spec
        return name, _draw_weight(index, shape, kind, key, bf16)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        return dict(ex.map(one, specs))


def make_workload(index: int, layers: Optional[int] = None, with_weights: bool = True) -> Workload:
    """The seeded workload `index` (1..5); `layers` truncates the tower (same weights per layer)."""
    cfg = tower_config(index)
    if layers is not None:
        cfg = cfg.with_layers(layers)
    items = []
    for i, (f, h, w) in enumerate(draw_items(index)):
        items.append(Item(_pixels(index, i, f, h, w), _grid(f, h, w)))
    weights = make_weights(index, cfg) if with_weights else {}
    return Workload(index, cfg, items, weights)


def make_custom_workload(cfg: TowerConfig, sizes: Sequence[Tuple[int, int, int]], seed: int,
                         with_weights: bool = True) -> Workload:
    """A workload of the given tower with item sizes (n_frames, H, W); streams keyed by `seed`."""
    items = [Item(_pixels(seed, i, f, h, w), _grid(f, h, w, cfg.temporal_patch, cfg.patch))
             for i, (f, h, w) in enumerate(sizes)]
    weights = make_weights(seed, cfg) if with_weights else {}
    return Workload(seed, cfg, items, weights)


def pack_pixels(items: Sequence[Item]) -> np.ndarray:
    """All items' frames back to back (item order, frame order, HWC rows): the library's pixel layout."""
    if not items:
        return np.zeros(0, dtype=np.uint8)
    return np.concatenate([np.ascontiguousarray(it.frames).reshape(-1) for it in items])
