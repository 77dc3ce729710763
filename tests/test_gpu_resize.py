"""Device resize to the 28-pixel grid (vit_resize_u8) against the CPU oracle, bit-exact:
off-grid sizes both ways, an on-grid image (identity), a large photo-sized image and a
multi-frame clip; then a resized image goes through the tower and matches the oracle
tower on the oracle-resized pixels."""

import numpy as np
import pytest
import torch

from oracle import resize as RS
from oracle import vit_oracle as O
from workloads import Item, Workload, make_weights, pack_pixels, tower_config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

from gpu_support import TowerRun, assert_encoder_tolerance  # noqa: E402
from multimodal_vlm_vision_amd import resize_side, resize_u8  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _device_resize(frames: np.ndarray) -> np.ndarray:
    F, H, W, _ = frames.shape
    dh, dw = resize_side(H), resize_side(W)
    assert (dh, dw) == (RS.resize_side(H), RS.resize_side(W))
    src = torch.from_numpy(np.ascontiguousarray(frames)).cuda()
    dst = torch.empty(F, dh, dw, 3, dtype=torch.uint8, device="cuda")
    resize_u8(src, H, W, F, dst)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 41, 47), (1, 69, 30), (1, 56, 84), (1, 1000, 700), (3, 500, 900),
                                   (1, 1, 1), (2, 13, 2000), (1, 30, 8000), (2, 8192, 40)])
def test_resize_bit_exact(shape):
    F, H, W = shape
    say(f"resize {shape}")
    g = np.random.default_rng(H * 7919 + W)
    x = g.integers(0, 256, size=(F, H, W, 3), dtype=np.uint8)
    got = _device_resize(x)
    assert np.array_equal(got, RS.resize(x))
    if H % 28 == 0 and W % 28 == 0:
        assert np.array_equal(got, x)


def test_resized_image_through_the_tower():
    cfg = tower_config(1)                                   # tiny tower, fp32 weights
    g = np.random.default_rng(3)
    raw = g.integers(0, 256, size=(1, 61, 90, 3), dtype=np.uint8)
    frames = _device_resize(raw)                            # 56 x 84 -> grid (1, 4, 6)
    say(f"resized {raw.shape[1:3]} -> {frames.shape[1:3]}, encoding")
    item = Item(frames, (1, frames.shape[1] // 14, frames.shape[2] // 14))
    wl = Workload(1, cfg, [item], make_weights(1, cfg))
    run = TowerRun(wl)
    got = run.encode()
    ref = O.forward_workload(wl)
    assert_encoder_tolerance(got, ref, what="resized image")
