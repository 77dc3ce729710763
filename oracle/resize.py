"""CPU oracle of the device resize to the 28-pixel grid (before the path).

TEST INFRASTRUCTURE ONLY (like ``vit_oracle``): only ``tests/`` may import it.
It shares no code with the HIP library.

The pages say the preprocessor resizes and pads images into pixel tensors
("vLLM multimodal inference | ViT performance optimisation", section 2.2) and
that CPU preprocessing caps serving throughput (SGLang PR #35349 report) but
fix neither the target size nor the interpolation.  The readings taken
here: each side goes to the nearest multiple of 28 pixels, half up, at
least 28; bilinear sampling with half-pixel centres, source coordinate
s = (d + 0.5) * S / D - 0.5 clamped to the image; weights in 11-bit fixed point
(w = round((s - floor(s)) * 2^11)), integer arithmetic, the result rounded
half up.  Written with integer arrays so it is exact.
"""

import numpy as np

Q = 11
ONE = 1 << Q


def resize_side(s: int) -> int:
    """Target of one side of s pixels: the nearest multiple of 28 (half up), at least 28."""
    return 28 * max((s + 14) // 28, 1)


def axis_weights(D: int, S: int):
    """(i0, i1, w) per output coordinate d < D of a side of S source pixels."""
    d = np.arange(D, dtype=np.int64)
    num = (2 * d + 1) * S - D            # s * 2D
    den = 2 * D
    pos = num > 0
    q = np.where(pos, num // den, 0)
    r = np.where(pos, num - q * den, 0)
    w = (r * ONE + den // 2) // den
    end = q >= S - 1
    i0 = np.where(end, S - 1, q)
    flat = end | ~pos
    i1 = np.where(flat, i0, i0 + 1)
    w = np.where(flat, 0, w)
    return i0, i1, w


def resize(frames: np.ndarray) -> np.ndarray:
    """[F][H][W][3] uint8 -> [F][resize_side(H)][resize_side(W)][3] uint8."""
    F, H, W, C = frames.shape
    dh, dw = resize_side(H), resize_side(W)
    y0, y1, wy = axis_weights(dh, H)
    x0, x1, wx = axis_weights(dw, W)
    f = frames.astype(np.int64)
    wx_ = wx[None, None, :, None]
    wy_ = wy[None, :, None, None]
    r0, r1 = f[:, y0], f[:, y1]
    top = (ONE - wx_) * r0[:, :, x0] + wx_ * r0[:, :, x1]
    bot = (ONE - wx_) * r1[:, :, x0] + wx_ * r1[:, :, x1]
    v = ((ONE - wy_) * top + wy_ * bot + (1 << (2 * Q - 1))) >> (2 * Q)
    return v.astype(np.uint8)
