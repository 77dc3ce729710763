"""Shape-bucketed graph (vit_graph_capture_bucket / vit_graph_launch_plan): one
capture for a capacity plan replays other batches of the same tower without
re-capture.  Each replay is bit-identical to eager encoding of that batch
(every kernel reads the batch sizes at run time; per-element arithmetic does
not depend on the tile configuration, which the capacity fixes) -- unless the
eager forward of that batch runs key-split attention units (bucketed graphs run
the plain unit lists), in which case the two are two summation orders of the
same softmax and agree to the encoder tolerance.  Two of the replays -- one
image and the video replayed alone -- are also compared with the oracle.  Also: a replay with leftovers of a larger batch in the workspace, a
batch over capacity, and a plain graph that cannot take plans."""

import numpy as np
import pytest
import torch

from workloads import make_custom_workload, make_workload, pack_pixels

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

from gpu_support import TowerRun, assert_encoder_tolerance  # noqa: E402
from oracle import vit_oracle as O  # noqa: E402
from multimodal_vlm_vision_amd.binding import VitError  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _grid(items):
    g = np.array([it.grid_thw for it in items], dtype=np.int32).reshape(-1, 3)
    f = np.array([it.n_frames for it in items], dtype=np.int32)
    return g, f


def _eager(tower, items, out_dim):
    plan = tower.plan(*_grid(items))
    px = torch.from_numpy(pack_pixels(items)).cuda()
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(plan.out_rows, out_dim, dtype=torch.float32, device="cuda")
    tower.encode(plan, px, ws, out)
    torch.cuda.synchronize()
    return plan, out.cpu().numpy()


def test_bucket_graph_replays_other_batches():
    # windowed and full-attention layers, RMSNorm, SwiGLU: every count the kernels read
    wl = make_workload(5, layers=8)
    run = TowerRun(wl)
    tower, cap, out_dim = run.tower, run.plan, wl.cfg.out_dim
    say(f"bucket capacity N={cap.n_patches}, {len(wl.items)} items")
    gws = torch.empty(cap.ws_bytes, dtype=torch.uint8, device="cuda")
    g = tower.capture_bucket(cap, gws)
    pix_off, out_off = g.pixels_ptr - gws.data_ptr(), g.out_ptr - gws.data_ptr()

    def replay(plan, items):
        px = torch.from_numpy(pack_pixels(items)).cuda()
        gws[pix_off:pix_off + px.numel()].copy_(px)
        g.launch_plan(plan)
        torch.cuda.synchronize()
        n = plan.out_rows
        return gws[out_off:out_off + n * out_dim * 4].view(torch.float32).reshape(n, out_dim).cpu().numpy()

    items = wl.items
    last = len(items) - 1
    batches = [("capacity batch", items), ("first 5 images", items[:5]), ("video alone", items[-1:]),
               ("images 3..8", items[3:9]), ("one small image", items[10:11]), ("capacity batch again", items)]
    # replays that are also compared with the oracle (whole output, float64)
    oracle_items = {"video alone": [last], "one small image": [10]}
    for name, sub in batches:
        plan, ref = _eager(tower, sub, out_dim)
        say(f"replay {name}: N={plan.n_patches}")
        got = replay(plan, sub)
        split = any(plan.attention_units(win)[1] > 0 for win in (False, True))
        if split:
            say(f"  eager runs key-split units: max |replay - eager| = {np.abs(got - ref).max():.3e}")
            assert_encoder_tolerance(got.astype(np.float64), ref.astype(np.float64),
                                     what=f"bucket replay vs eager (key splits), {name}")
        else:
            assert np.array_equal(got, ref), f"{name}: bucket replay differs from eager"
        if name in oracle_items:
            want = O.forward_workload(wl, items=oracle_items[name])
            assert_encoder_tolerance(got.astype(np.float64), want, what=f"bucket replay, {name}")

    # the plain launch replays the last uploaded batch
    g.launch()
    torch.cuda.synchronize()
    n = cap.out_rows
    got = gws[out_off:out_off + n * out_dim * 4].view(torch.float32).reshape(n, out_dim).cpu().numpy()
    if any(cap.attention_units(win)[1] > 0 for win in (False, True)):
        assert_encoder_tolerance(got.astype(np.float64), run.encode().astype(np.float64),
                                 what="plain launch vs eager (key splits)")
    else:
        assert np.array_equal(got, run.encode())

    # over capacity: more patches than captured
    big = tower.plan(*_grid(items + items[:1]))
    with pytest.raises(VitError, match="exceeds the bucket"):
        g.launch_plan(big)
    # a different tower configuration
    other = make_custom_workload(wl.cfg.with_layers(2), [(1, 56, 56)], seed=7, with_weights=False)
    # (plans carry the tower configuration; a two-layer plan does not fit this graph)
    from multimodal_vlm_vision_amd import VisionTower
    t2 = VisionTower(other.cfg)
    p2 = t2.plan(*_grid(other.items))
    with pytest.raises(VitError, match="another tower"):
        g.launch_plan(p2)
    g.close()


def test_plain_graph_rejects_plans():
    run = TowerRun(make_workload(1))
    gws = torch.empty(run.plan.ws_bytes, dtype=torch.uint8, device="cuda")
    g = run.tower.capture(run.plan, gws)
    with pytest.raises(VitError, match="capture_bucket"):
        g.launch_plan(run.plan)
    g.close()
