"""Vision-embedding cache (vit_encode_cached, vit_pixel_keys) on the GPU:

* the device pixel content keys equal the CPU oracle's (bit-exact);
* a batch encoded through the cache equals plain encoding, bit for bit, on a
  cold cache (all misses), a warm one (all hits) and mixes of cached, changed
  and repeated items -- when the batch's plain encoding runs no key-split
  attention units (the cache encodes its misses without them); otherwise the
  two agree to the encoder tolerance (the same softmax summed in another order);
* a small arena evicts first-in first-out and stays correct.
"""

import numpy as np
import pytest
import torch

from oracle import pixel_key as PK
from workloads import make_workload, pack_pixels

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

from gpu_support import TowerRun, assert_encoder_tolerance  # noqa: E402
from multimodal_vlm_vision_amd import EmbeddingCache  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _grid(items):
    return (np.array([it.grid_thw for it in items], dtype=np.int32).reshape(-1, 3),
            np.array([it.n_frames for it in items], dtype=np.int32))


class Batch:
    def __init__(self, tower, items, out_dim):
        self.items = items
        self.plan = tower.plan(*_grid(items))
        self.px = torch.from_numpy(pack_pixels(items)).cuda()
        self.ws = torch.empty(self.plan.ws_bytes, dtype=torch.uint8, device="cuda")
        self.out = torch.empty(self.plan.out_rows, out_dim, dtype=torch.float32, device="cuda")

    def plain(self, tower):
        tower.encode(self.plan, self.px, self.ws, self.out)
        torch.cuda.synchronize()
        return self.out.cpu().numpy().copy()

    def cached(self, tower, cache):
        self.out.fill_(float("nan"))
        hits = tower.encode_cached(cache, self.plan, self.px, self.ws, self.out)
        torch.cuda.synchronize()
        return hits, self.out.cpu().numpy().copy()


def same(got, ref, batch, what):
    """Bit-identical unless the batch's plain encoding runs key-split units."""
    if any(batch.plan.attention_units(w)[1] > 0 for w in (False, True)):
        say(f"{what}: plain encoding runs key-split units, max diff {np.abs(got - ref).max():.3e}")
        assert_encoder_tolerance(got.astype(np.float64), ref.astype(np.float64), what=what)
    else:
        assert np.array_equal(got, ref), what


@pytest.fixture(scope="module")
def run():
    return TowerRun(make_workload(3, layers=2))   # 8 images of mixed sizes, 2 layers


def test_device_pixel_keys_match_oracle(run):
    say("pixel keys")
    b = Batch(run.tower, run.wl.items, run.cfg.out_dim)
    got = run.tower.pixel_keys(b.plan, b.px, b.ws)
    want = np.array([PK.item_key(it.frames) for it in run.wl.items], dtype=np.uint64)
    assert np.array_equal(got, want)
    # the video item of workload 4 (16 frames) as well
    vid = make_workload(4, with_weights=False).items
    vb = Batch(run.tower, vid, run.cfg.out_dim)
    assert np.array_equal(run.tower.pixel_keys(vb.plan, vb.px, vb.ws),
                          np.array([PK.item_key(it.frames) for it in vid], dtype=np.uint64))


def test_cached_encode_equals_plain(run):
    t, items, od = run.tower, run.wl.items, run.cfg.out_dim
    arena = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    cache = EmbeddingCache(t, arena)
    full = Batch(t, items, od)
    ref = full.plain(t)
    say("cold cache")
    hits, got = full.cached(t, cache)
    assert hits == 0
    same(got, ref, full, "cold cache")
    assert cache.stats()[0] == len(items)
    say("warm cache")
    hits, got = full.cached(t, cache)
    assert hits == len(items)
    same(got, ref, full, "warm cache")

    # cached items, one changed pixel (a different key), a repeat inside the batch
    changed = type(items[3])(items[3].frames.copy(), items[3].grid_thw)
    changed.frames[0, 5, 7, 2] ^= 0x40
    mix = [items[5], changed, items[0], items[5], items[2]]
    mb = Batch(t, mix, od)
    ref_mix = mb.plain(t)
    say("mixed batch")
    hits, got = mb.cached(t, cache)
    assert hits == 4
    same(got, ref_mix, mb, "mixed batch")
    cache.close()


def test_small_arena_evicts_fifo(run):
    t, items, od = run.tower, run.wl.items, run.cfg.out_dim
    full = Batch(t, items, od)
    ref = full.plain(t)
    row_bytes = od * 4
    sizes = [it.n_patches // 4 * row_bytes for it in items]
    arena_bytes = (max(sizes) * 2 + 255) // 256 * 256 + 256
    arena = torch.empty(arena_bytes, dtype=torch.uint8, device="cuda")
    cache = EmbeddingCache(t, arena)
    say(f"small arena {arena_bytes} bytes")
    hits, got = full.cached(t, cache)
    assert hits == 0
    same(got, ref, full, "small arena, cold")
    n, used = cache.stats()
    assert 1 <= n < len(items) and used <= arena_bytes
    hits, got = full.cached(t, cache)
    same(got, ref, full, "small arena, again")
    # the last item inserted is still there
    last = Batch(t, items[-1:], od)
    h1, g1 = last.cached(t, cache)
    same(g1, last.plain(t), last, "last item")
    cache.close()
