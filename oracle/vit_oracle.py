"""CPU oracle for the Qwen2-VL / Qwen2.5-VL-style vision-tower forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the only common import is the seeded input generator ``workloads``.

It is a plain, slow transcription of what the pages say the tower computes,
in float64 by default (``dtype=np.float32`` is accepted for large cases):

1. rescale + normalise uint8 pixels into the tower dtype (bfloat16) -- vLLM
   PR #55370 report, "implementation breakdown" (the tower's first step is the
   fused input norm that takes integer pixels and returns tower-dtype values)
   and the review highlights (uint8 values are exact in bfloat16);
2. cut 14x14 patches, keep each 2x2 merge unit contiguous, flatten to
   (c, tau, i, j) rows -- "vLLM multimodal inference | ViT performance
   optimisation", sections 2.2 (encoding step 1) and 3.2;
3. patch embedding = a 3D convolution whose kernel equals its stride, done
   as one matrix product (same blog, section 3.2);
4. 2D rotary positions: per-patch (hpos, wpos) in merge order, the first
   half of the angles from the row position and the second half from the
   column position (same blog, section 3.3);
5. L transformer blocks: norm -> qkv -> RoPE on q, k -> attention that never
   crosses an item boundary (cu_seqlens, same blog, section 3.4; windows in
   window-attention layers, section 3.3) -> out-proj + residual -> norm ->
   MLP + residual (sections 2.2 and 3.1);
6. the patch merger: each 2x2 group of patch features -> one token through an
   MLP projector (section 2.2, encoding step 4).

Readings where the pages are silent:
x/255 as the rescale; bfloat16 round-to-nearest-even of the exact value; row
order (dh, dw) inside a merge unit and t-major across frames; feature order
(c, tau, i, j); an image's single frame duplicated to the temporal patch;
RoPE base 10000 with rotate-half pairing (k, k + head_dim/2); attention scale
1/sqrt(head_dim); exact-erf GELU; LayerNorm with biased variance; one
attention segment per item (a whole video is one segment); 112 px windows of
8x8 patches per frame tiled from the top-left; merger pre-norm of the block
norm kind, hidden width 4*d, GELU.

Parity unpinned (conventions every invariant accepts; fixed only by the
readings above): the RoPE pairing convention and base, the GELU variant,
which linears carry biases, and per-item rather than per-frame video
segments.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf
from threadpoolctl import threadpool_limits

# ----------------------------------------------------------------------------
# scheduling only: independent rows and independent (segment, query block)
# pieces of attention run on a thread pool (NumPy and SciPy release the GIL
# inside their loops).  Every element is computed by the same operations in
# the same order as in a serial run; only which thread computes it changes.
# ----------------------------------------------------------------------------

_POOL: Optional[ThreadPoolExecutor] = None
_ROW_BLOCK = 2048


def _threads() -> int:
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:   # the CPU share this process is given
        n = min(n, int(cap))
    return max(1, n)


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(_threads())
    return _POOL


def _rowwise(f: Callable[[np.ndarray], np.ndarray], x: np.ndarray) -> np.ndarray:
    """f applied to x, where f acts on each row (leading index) on its own."""
    if x.ndim < 2 or x.shape[0] <= _ROW_BLOCK or _threads() == 1:
        return f(x)
    parts = list(_pool().map(f, [x[i:i + _ROW_BLOCK] for i in range(0, x.shape[0], _ROW_BLOCK)]))
    return np.concatenate(parts, axis=0)


# ----------------------------------------------------------------------------
# 1. normalisation
# ----------------------------------------------------------------------------


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits.  frexp gives v = m * 2**e with
    0.5 <= |m| < 1; m * 256 then has exactly 8 integer bits and rint rounds
    it half-to-even.  (Subnormal and overflow ranges never occur here.)
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def normalize_table(mean: Sequence[float], std: Sequence[float]) -> np.ndarray:
    """[3][256] float64: bf16(((x / 255) - mean_c) / std_c) for every uint8 x.

    mean_c and std_c are taken as float32 numbers, the precision of the
    configured parameters.  Output dtype is the tower dtype (bfloat16), so
    every value is rounded once from (a float64 evaluation of) the exact
    quotient.
    """
    x = np.arange(256, dtype=np.float64)
    rows = []
    for c in range(3):
        m = float(np.float32(mean[c]))
        s = float(np.float32(std[c]))
        rows.append(bf16_round(((x / 255.0) - m) / s))
    return np.stack(rows)


# ----------------------------------------------------------------------------
# 2. patchify (merge-unit order) and 3. patch embedding
# ----------------------------------------------------------------------------


def item_clip(frames: np.ndarray, temporal_patch: int = 2) -> np.ndarray:
    """The item's frames, an image's single frame repeated temporal_patch times."""
    if frames.shape[0] == 1:
        return np.repeat(frames, temporal_patch, axis=0)
    return frames


def patch_positions(grid_thw: np.ndarray, merge: int = 2) -> Dict[str, np.ndarray]:
    """Per patch row, in merge order: item, temporal index t, hpos, wpos.

    Rows of an item run over t, then merge-block row bh, merge-block column
    bw, then (dh, dw) inside the block, so every 2x2 merge unit is 4
    consecutive rows; the T frames of an item repeat the same 2D positions.
    """
    item, tt, hp, wp = [], [], [], []
    for n, (t, h, w) in enumerate(np.asarray(grid_thw).reshape(-1, 3)):
        for ti in range(t):
            for bh in range(h // merge):
                for bw in range(w // merge):
                    for dh in range(merge):
                        for dw in range(merge):
                            item.append(n)
                            tt.append(ti)
                            hp.append(bh * merge + dh)
                            wp.append(bw * merge + dw)
    return {"item": np.array(item, dtype=np.int64), "t": np.array(tt, dtype=np.int64),
            "hpos": np.array(hp, dtype=np.int64), "wpos": np.array(wp, dtype=np.int64)}


def patchify(items_frames: Sequence[np.ndarray], grid_thw: np.ndarray, table: np.ndarray,
             temporal_patch: int = 2, patch: int = 14, merge: int = 2) -> np.ndarray:
    """flatten_patches [N][3 * tp * p * p] (float64 holding bf16 values), rows in merge order."""
    rows = []
    for frames, (t, h, w) in zip(items_frames, np.asarray(grid_thw).reshape(-1, 3)):
        clip = item_clip(frames, temporal_patch)                   # [F][H][W][3] uint8
        normed = np.stack([table[c][clip[..., c]] for c in range(3)], axis=-1)
        for ti in range(t):
            for bh in range(h // merge):
                for bw in range(w // merge):
                    for dh in range(merge):
                        for dw in range(merge):
                            ph, pw = bh * merge + dh, bw * merge + dw
                            blk = normed[ti * temporal_patch:(ti + 1) * temporal_patch,
                                         ph * patch:(ph + 1) * patch,
                                         pw * patch:(pw + 1) * patch, :]    # [tau][i][j][c]
                            rows.append(blk.transpose(3, 0, 1, 2).reshape(-1))  # (c, tau, i, j)
    width = 3 * temporal_patch * patch * patch
    return np.array(rows, dtype=np.float64).reshape(-1, width)


def patch_embed(x: np.ndarray, w_pe: np.ndarray) -> np.ndarray:
    """The stride-equals-kernel conv as one product: [N][1176] @ [1176][d]."""
    return x @ w_pe.reshape(w_pe.shape[0], -1).T


# ----------------------------------------------------------------------------
# 4. 2D rotary position embedding
# ----------------------------------------------------------------------------


def rope_angles(hpos: np.ndarray, wpos: np.ndarray, head_dim: int, theta: float = 10000.0,
                dtype=np.float64) -> np.ndarray:
    """[N][head_dim/2] rotation angles: the first half from hpos, the second from wpos.

    rotary_dim = head_dim / 2 angles per head; each axis gets rotary_dim / 2
    frequencies theta ** (-2 j / rotary_dim).
    """
    rotary_dim = head_dim // 2
    nfreq = rotary_dim // 2
    inv = theta ** (-2.0 * np.arange(nfreq, dtype=np.float64) / rotary_dim)
    a_h = np.outer(hpos.astype(np.float64), inv)
    a_w = np.outer(wpos.astype(np.float64), inv)
    return np.concatenate([a_h, a_w], axis=1).astype(dtype)


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on x [N][H][head_dim]: pair (k, k + head_dim/2) turns by angle k."""
    r = x.shape[-1] // 2
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    if x.ndim == 3 and x.shape[0] > _ROW_BLOCK and _threads() > 1:
        blocks = range(0, x.shape[0], _ROW_BLOCK)
        return np.concatenate(list(_pool().map(
            lambda i: apply_rope(x[i:i + _ROW_BLOCK], angles[i:i + _ROW_BLOCK]), blocks)), axis=0)
    x1, x2 = x[..., :r], x[..., r:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    def f(x):
        mu = x.mean(axis=-1, keepdims=True)
        var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
        return (x - mu) / np.sqrt(var + eps) * g + b
    return _rowwise(f, x)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    return _rowwise(lambda x: x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * g, x)


def gelu(x: np.ndarray) -> np.ndarray:
    return _rowwise(lambda x: 0.5 * x * (1.0 + erf(x / math.sqrt(2.0))), x)


def silu(x: np.ndarray) -> np.ndarray:
    return _rowwise(lambda x: x / (1.0 + np.exp(-x)), x)


def norm(x: np.ndarray, weights: Dict[str, np.ndarray], prefix: str, kind: str, eps: float,
         dtype=np.float64) -> np.ndarray:
    g = weights[prefix + ".g"].astype(dtype)
    if kind == "layer":
        return layer_norm(x, g, weights[prefix + ".b"].astype(dtype), eps)
    return rms_norm(x, g, eps)


# ----------------------------------------------------------------------------
# 5. attention segments and attention
# ----------------------------------------------------------------------------


def item_segments(pos: Dict[str, np.ndarray]) -> List[np.ndarray]:
    """One segment per item: cu_seqlens isolation, no other mask."""
    return [np.nonzero(pos["item"] == n)[0] for n in np.unique(pos["item"])]


def window_segments(pos: Dict[str, np.ndarray], window_patches: int) -> List[np.ndarray]:
    """Segments of window-attention layers, as index sets in original row order.

    A window is (item, frame t, hpos // W, wpos // W) for W = window_px / patch
    patches per side, tiled from the top-left of each frame; edge windows are
    truncated.
    """
    key = np.stack([pos["item"], pos["t"], pos["hpos"] // window_patches,
                    pos["wpos"] // window_patches], axis=1)
    _, inverse = np.unique(key, axis=0, return_inverse=True)
    inverse = inverse.reshape(-1)
    order = np.argsort(inverse, kind="stable")
    bounds = np.flatnonzero(np.diff(inverse[order])) + 1
    return np.split(order, bounds)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, segments: Sequence[np.ndarray],
              rows: Optional[np.ndarray] = None, chunk: int = 256) -> np.ndarray:
    """softmax(Q K^T / sqrt(head_dim)) V inside each segment, per head.

    q, k, v: [N][H][head_dim].  If `rows` is given only those query rows are
    produced (returned in the order of `rows`); every segment still uses all
    of its keys.
    """
    n_rows, heads, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    out = np.zeros_like(q) if rows is None else np.zeros((len(rows), heads, hd), dtype=q.dtype)
    where = None
    if rows is not None:
        where = np.full(n_rows, -1, dtype=np.int64)
        where[rows] = np.arange(len(rows))
    tasks = []
    for seg in segments:
        qrows = seg if where is None else seg[where[seg] >= 0]
        for c0 in range(0, qrows.size, chunk):
            tasks.append((seg, qrows[c0:c0 + chunk]))

    def one(task):
        seg, qr = task
        kt = np.ascontiguousarray(k[seg].transpose(1, 2, 0))          # [H][hd][n]
        vs = np.ascontiguousarray(v[seg].transpose(1, 0, 2))          # [H][n][hd]
        qh = np.ascontiguousarray(q[qr].transpose(1, 0, 2))           # [H][nq][hd]
        s = qh @ kt                                                   # [H][nq][n]
        s *= scale
        s -= s.max(axis=-1, keepdims=True)
        p = np.exp(s, out=s)
        p /= p.sum(axis=-1, keepdims=True)
        o = (p @ vs).transpose(1, 0, 2)                               # [nq][H][hd]
        if where is None:
            out[qr] = o
        else:
            out[where[qr]] = o

    if len(tasks) > 1 and _threads() > 1:
        # one BLAS thread per task: the pieces themselves run in parallel
        with threadpool_limits(limits=1, user_api="blas"):
            list(_pool().map(one, tasks))
    else:
        for t in tasks:
            one(t)
    return out


def layer_segments(layer: int, cfg, pos: Dict[str, np.ndarray]) -> List[np.ndarray]:
    if cfg.window_px and layer not in cfg.full_attn_layers:
        return window_segments(pos, cfg.window_px // cfg.patch)
    return item_segments(pos)


# ----------------------------------------------------------------------------
# one block
# ----------------------------------------------------------------------------


def _w(weights, name, dtype):
    return weights[name].astype(dtype)


def block(r: np.ndarray, weights: Dict[str, np.ndarray], layer: int, cfg, angles: np.ndarray,
          segments: Sequence[np.ndarray], rows: Optional[np.ndarray] = None,
          trace: Optional[dict] = None) -> np.ndarray:
    """One pre-norm block on the residual stream r [N][d].

    With `rows`, only those rows of the block output are computed (keys and
    values still come from every row); the result has len(rows) rows.
    """
    dt = r.dtype
    d, heads = cfg.hidden, cfg.heads
    hd = d // heads
    p = f"blk{layer}"
    h = norm(r, weights, p + ".n1", cfg.norm_kind, cfg.norm_eps, dt)
    qkv = h @ _w(weights, p + ".qkv.w", dt).T + _w(weights, p + ".qkv.b", dt)
    q = qkv[:, 0 * d:1 * d].reshape(-1, heads, hd)
    k = qkv[:, 1 * d:2 * d].reshape(-1, heads, hd)
    v = qkv[:, 2 * d:3 * d].reshape(-1, heads, hd)
    q = apply_rope(q, angles)
    k = apply_rope(k, angles)
    o = attention(q, k, v, segments, rows=rows).reshape(-1, d)
    r_sel = r if rows is None else r[rows]
    r1 = r_sel + o @ _w(weights, p + ".proj.w", dt).T + _w(weights, p + ".proj.b", dt)
    h2 = norm(r1, weights, p + ".n2", cfg.norm_kind, cfg.norm_eps, dt)
    if cfg.mlp_kind == "gelu":
        a = gelu(h2 @ _w(weights, p + ".fc1.w", dt).T + _w(weights, p + ".fc1.b", dt))
        m = a @ _w(weights, p + ".fc2.w", dt).T + _w(weights, p + ".fc2.b", dt)
    else:
        gt = h2 @ _w(weights, p + ".gate.w", dt).T + _w(weights, p + ".gate.b", dt)
        up = h2 @ _w(weights, p + ".up.w", dt).T + _w(weights, p + ".up.b", dt)
        a = silu(gt) * up
        m = a @ _w(weights, p + ".down.w", dt).T + _w(weights, p + ".down.b", dt)
    out = r1 + m
    if trace is not None:
        trace.update(h1=h, q=q, k=k, v=v, attn=o, r_attn=r1, h2=h2, act=a, out=out)
    return out


# ----------------------------------------------------------------------------
# 6. patch merger
# ----------------------------------------------------------------------------


def merger(r: np.ndarray, weights: Dict[str, np.ndarray], cfg, trace: Optional[dict] = None
           ) -> np.ndarray:
    """Norm each patch row, join each merge unit's 4 rows into one vector, MLP projector."""
    dt = r.dtype
    u = norm(r, weights, "mrg.nq", cfg.norm_kind, cfg.norm_eps, dt)
    unit = cfg.merge * cfg.merge
    u = u.reshape(-1, unit * cfg.hidden)
    z1 = gelu(u @ _w(weights, "mrg.fc1.w", dt).T + _w(weights, "mrg.fc1.b", dt))
    z = z1 @ _w(weights, "mrg.fc2.w", dt).T + _w(weights, "mrg.fc2.b", dt)
    if trace is not None:
        trace.update(u=u, hidden=z1, out=z)
    return z


# ----------------------------------------------------------------------------
# whole tower
# ----------------------------------------------------------------------------


def forward(items_frames: Sequence[np.ndarray], grid_thw: np.ndarray, cfg,
            weights: Dict[str, np.ndarray], dtype=np.float64, layers: Optional[int] = None,
            trace: Optional[dict] = None, progress: Optional[Callable[[int], None]] = None
            ) -> np.ndarray:
    """uint8 frames -> merged embeddings [N/4][out_dim], items in order.

    trace (optional dict) receives: "x" (normalised patches), "r0" (patch
    embedding), "r" (list of block outputs), "merger" (merger intermediates).
    progress (optional) is called with each layer index once that block is done.
    """
    n_layers = cfg.layers if layers is None else layers
    table = normalize_table(cfg.mean, cfg.std)
    x = patchify(items_frames, grid_thw, table, cfg.temporal_patch, cfg.patch, cfg.merge)
    pos = patch_positions(grid_thw, cfg.merge)
    angles = rope_angles(pos["hpos"], pos["wpos"], cfg.head_dim, cfg.rope_theta, dtype)
    r = patch_embed(x.astype(dtype), weights["pe.w"].astype(dtype))
    if trace is not None:
        trace.update(x=x, r0=r.copy(), r=[], pos=pos)
    for l in range(n_layers):
        r = block(r, weights, l, cfg, angles, layer_segments(l, cfg, pos))
        if trace is not None:
            trace["r"].append(r.copy())
        if progress is not None:
            progress(l)
    mt = {} if trace is not None else None
    out = merger(r, weights, cfg, trace=mt)
    if trace is not None:
        trace["merger"] = mt
    return out


def forward_workload(wl, dtype=np.float64, layers: Optional[int] = None,
                     items: Optional[Sequence[int]] = None, trace: Optional[dict] = None,
                     progress: Optional[Callable[[int], None]] = None) -> np.ndarray:
    """forward() on a `workloads.Workload`, optionally on a subset of its items."""
    sel = list(range(len(wl.items))) if items is None else list(items)
    frames = [wl.items[i].frames for i in sel]
    grid = np.array([wl.items[i].grid_thw for i in sel], dtype=np.int64).reshape(-1, 3)
    return forward(frames, grid, wl.cfg, wl.weights, dtype=dtype, layers=layers, trace=trace,
                   progress=progress)
