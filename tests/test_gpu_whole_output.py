"""Whole-output parity of the three 32-layer workloads, through the path the bench times.

Each workload's complete output (every item, every merged token, every column) comes from
the captured whole-encoder graph (vit_graph_capture + vit_graph_launch, uint8 pixels written
into the graph's input region) and is compared element by element with the CPU oracle in
float32 on the same seeded inputs:

* the 8-image mixed-resolution batch (17,624 patches, item segments);
* the 16-frame 504x896 video, one 18,432-token attention segment;
* the Qwen2.5-shaped batch of 12 images and an 8-frame video (15,384 patches, RMSNorm,
  SwiGLU, 112 px windows with whole-item attention in layers 7, 15, 23 and 31).

Bar: max |g - r| <= 2e-2 and sum |g - r| / sum |r| <= 5e-3 over the whole output.  Each
item's own figures are printed as well.  The oracle's long runs report each finished layer
on stderr (and in the file VIT_TEST_PROGRESS names, when set).
"""

import time

import numpy as np
import pytest
import torch

from oracle import vit_oracle as O
from workloads import make_workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

from gpu_support import TowerRun, assert_encoder_tolerance, per_item_errors, progress_log, rel_err  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    progress_log(msg)


@pytest.mark.parametrize("idx", [3, 4, 5])
def test_whole_output_through_graph_matches_oracle(idx):
    wl = make_workload(idx)
    run = TowerRun(wl)
    say(f"workload {idx} ({wl.cfg.name}): N={run.n}, {len(wl.items)} items, graph replay")
    got = run.graph_encode(replays=2)
    del run
    torch.cuda.empty_cache()
    t0 = time.time()
    ref = O.forward_workload(wl, dtype=np.float32,
                             progress=lambda l: progress_log(f"workload {idx}: oracle layer {l} done "
                                                             f"({time.time() - t0:.0f} s)"))
    say(f"workload {idx}: oracle (float32, {O._threads()} threads) {time.time() - t0:.1f} s")
    for i, (ma, mr) in enumerate(per_item_errors(got, ref, wl.items)):
        say(f"workload {idx} item {i} grid {wl.items[i].grid_thw}: max_abs={ma:.3e} mean_rel={mr:.3e}")
    say(f"workload {idx} whole output: max_abs={float(np.abs(got - ref).max()):.3e} "
        f"mean_rel={rel_err(got, ref):.3e}")
    assert_encoder_tolerance(got, ref, what=f"workload {idx} whole output (graph)")
