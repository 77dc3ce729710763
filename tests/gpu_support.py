"""Shared helpers of the GPU tests: run a workload through the C ABI with
torch-allocated device buffers, fetch intermediate stages, and map the
library's internal row order back to merge order.  (Not a test module.)"""

from __future__ import annotations

import numpy as np
import torch

from multimodal_vlm_vision_amd import VisionTower
from workloads import pack_pixels


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


class TowerRun:
    def __init__(self, wl, activation_precision: str = "f16"):
        self.wl = wl
        self.prec = activation_precision
        cfg = wl.cfg
        self.cfg = cfg
        self.S = 2 if activation_precision in ("bf16x2", "bf16f8") else 1
        self.mlp_pad = (cfg.mlp_dim + 63) // 64 * 64
        self.tower = VisionTower(cfg, activation_precision=activation_precision)
        self.tower.load_weights(wl.weights)
        self.tower.finalize()
        self.plan = self.tower.plan(wl.grid_thw, wl.n_frames)
        self.n = self.plan.n_patches
        self.perm = self.plan.row_order().astype(np.int64)          # internal row -> merge-order row
        px = pack_pixels(wl.items)
        self.pixels = torch.from_numpy(px).cuda() if px.size else torch.empty(0, dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(max(self.plan.ws_bytes, 256), dtype=torch.uint8, device="cuda")
        self.out = torch.empty(max(self.plan.out_rows, 1), cfg.out_dim, dtype=torch.float32, device="cuda")

    def encode(self) -> np.ndarray:
        self.tower.encode(self.plan, self.pixels, self.ws, self.out)
        torch.cuda.synchronize()
        return self.out[: self.plan.out_rows].cpu().numpy().astype(np.float64)

    def graph_encode(self, replays: int = 2) -> np.ndarray:
        """The output of the captured whole-encoder graph (vit_graph_capture, then
        vit_graph_launch): the pixels are written into the graph's uint8 input region and the
        graph is replayed `replays` times, with eager work between replays; every replay must
        give the same bytes.  Returns the first replay's output."""
        gws = torch.empty(self.plan.ws_bytes, dtype=torch.uint8, device="cuda")
        g = self.tower.capture(self.plan, gws)
        try:
            off = g.pixels_ptr - gws.data_ptr()
            gws[off:off + self.pixels.numel()].copy_(self.pixels)
            out_off = g.out_ptr - gws.data_ptr()
            rows, cols = self.plan.out_rows, self.cfg.out_dim
            first = None
            for rep in range(replays):
                g.launch()
                torch.cuda.synchronize()
                got = gws[out_off:out_off + rows * cols * 4].view(torch.float32).reshape(rows, cols).cpu().numpy()
                if first is None:
                    first = got
                else:
                    assert np.array_equal(got, first), f"graph replay {rep} differs from replay 0"
                if rep + 1 < replays:
                    self.encode()          # eager work on another workspace between replays
        finally:
            g.close()
            del gws
        return first.astype(np.float64)

    def _join(self, a: np.ndarray, width: int, keep: int) -> np.ndarray:
        """[rows][S*width] stored activations -> values (hi + lo when split), first `keep` columns."""
        if self.S == 2:
            return a[:, :keep] + a[:, width:width + keep]
        return a[:, :keep]

    def stage(self, layer: int, step: int) -> np.ndarray:
        """An intermediate as values (hi + lo joined), rows in *merge order* (token-major)."""
        c, n, S = self.cfg, self.n, self.S
        d, h, hd = c.hidden, c.heads, c.head_dim
        L = c.layers
        a16 = torch.float16 if self.prec == "f16" else torch.bfloat16   # activations, q, k, v
        if layer == -1:
            shape, dt = ((n, 1176), torch.bfloat16) if step == 0 else ((n, d), torch.float32)
        elif layer == L:
            shape, dt = {1: ((n, S * d), a16), 2: ((n // 4, S * 4 * d), a16),
                         3: ((n // 4, c.out_dim), torch.float32)}[step]
        else:
            shape, dt = {1: ((n, S * d), a16), 2: ((h, n, hd), a16),
                         3: ((h, n, hd), a16), 4: ((h, hd, n), a16),
                         5: ((n, S * d), a16), 6: ((n, d), torch.float32),
                         7: ((n, S * d), a16), 8: ((n, S * self.mlp_pad), a16),
                         9: ((n, d), torch.float32)}[step]
        dst = torch.empty(shape, dtype=dt, device="cuda")
        self.tower.debug_stage(self.plan, self.pixels, self.ws, layer, step, dst)
        torch.cuda.synchronize()
        a = to_np(dst)
        if (layer == L and step == 1) or (0 <= layer < L and step in (1, 5, 7)):
            a = self._join(a, d, d)
        elif 0 <= layer < L and step == 8:
            a = self._join(a, self.mlp_pad, c.mlp_dim)
        elif layer == L and step == 2:
            a = self._join(a, 4 * d, 4 * d)
        if layer != -1 and layer != c.layers and step in (2, 3):
            a = a.transpose(1, 0, 2)                  # -> [n][heads][hd]
        if layer != -1 and layer != c.layers and step == 4:
            a = a.transpose(2, 0, 1)                  # -> [n][heads][hd]
        if layer == c.layers and step == 3:
            return a                                  # the output is scattered to item order by the library
        out = np.empty_like(a)
        if layer == c.layers and step == 2:
            out[self.perm[0::4] // 4] = a             # merged rows follow the internal unit order
        else:
            out[self.perm] = a
        return out


def progress_log(msg: str):
    """A progress line of a long test step (test output is captured until a test ends): written
    to the process's own stderr, past pytest's capture, and appended to the file named by the
    VIT_TEST_PROGRESS environment variable when that is set."""
    import os
    import sys
    import time
    line = f"{time.strftime('%H:%M:%S')} {msg}\n"
    sys.__stderr__.write(line)
    sys.__stderr__.flush()
    path = os.environ.get("VIT_TEST_PROGRESS")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(line)


def per_item_errors(got: np.ndarray, ref: np.ndarray, items) -> list:
    """(max_abs, mean_rel) of each item's merged rows (output rows are in item order)."""
    out, r0 = [], 0
    for it in items:
        r1 = r0 + it.n_patches // 4
        g, r = got[r0:r1], ref[r0:r1]
        out.append((float(np.abs(g - r).max()), rel_err(g, r)))
        r0 = r1
    return out


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).sum() / max(np.abs(ref).sum(), 1e-300))


def assert_encoder_tolerance(got: np.ndarray, ref: np.ndarray, max_abs=2e-2, mean_rel=5e-3, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma = float(np.abs(got - ref).max())
    mr = rel_err(got, ref)
    print(f"[parity] {what}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
    assert ma <= max_abs and mr <= mean_rel, f"{what}: max_abs={ma:.3e} mean_rel={mr:.3e}"


def unit(run) -> float:
    """Relative rounding unit of the library's 16-bit activations: 2^-11 for float16, 2^-8 for
    bfloat16 (one unit of the last place at the bottom of a binade)."""
    return 2.0 ** -11 if run.prec == "f16" else 2.0 ** -8


def assert_close_bf16(got: np.ndarray, ref: np.ndarray, rel=2.0 ** -7, abs_=1e-6, what="", extra=0.0):
    """Element-wise |got - ref| <= abs + rel * |ref| + extra (16-bit output rounding plus fp32
    accumulation; extra: a per-element bound of a known approximation, e.g. the e4m3 residual
    products)."""
    err = np.abs(got - ref)
    bound = abs_ + rel * np.abs(ref) + extra
    bad = err > bound
    print(f"[parity] {what}: max_abs={err.max():.3e} worst_ratio={(err / bound).max():.3f}", flush=True)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"


def f8_extra(run, x: np.ndarray, w: np.ndarray):
    """Per-element bound on how far the bf16 + e4m3-residual product x @ w.T may sit from the
    exact product of the values x the library reports (hi + residual): the residual is at most
    2^-8 |x| (times 1 + 2^-4 after its own e4m3 rounding) and meets an e4m3 copy of w, whose
    per-row power-of-two scale keeps every weight above 2^-6 of its row's largest one normal
    (relative error <= 2^-4); a factor 2 covers the smaller (subnormal) weights and the fp8
    MFMA's own rounding (~4e-5 of the residual term).  0 for the other precisions."""
    if run.prec != "bf16f8":
        return 0.0
    return 2.0 ** -11 * (np.abs(x) @ np.abs(w).T)
