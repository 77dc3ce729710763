"""Streams and contexts: an encode issued on a side stream gives the same bytes as one on the
default stream, and two towers with different weights and batches, encoded alternately on two
streams (their kernels free to overlap), each give the bytes they give alone."""

import numpy as np
import pytest
import torch

from workloads import make_custom_workload, tower_config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

from gpu_support import TowerRun  # noqa: E402


def _encode(run, stream):
    run.tower.encode(run.plan, run.pixels, run.ws, run.out, stream)


def test_side_stream_encode_matches_default_stream():
    wl = make_custom_workload(tower_config(2).with_layers(2), [(1, 224, 336), (2, 112, 112)], seed=89)
    run = TowerRun(wl)
    ref = run.encode()
    run.out.fill_(float("nan"))
    side = torch.cuda.Stream()           # default priority
    torch.cuda.synchronize()
    _encode(run, side)
    side.synchronize()
    got = run.out[: run.plan.out_rows].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)


def test_two_towers_on_two_streams():
    wa = make_custom_workload(tower_config(2).with_layers(2), [(1, 224, 224), (1, 112, 336)], seed=97)
    wb = make_custom_workload(tower_config(1), [(1, 56, 84), (4, 56, 56), (1, 112, 56)], seed=101)
    ra, rb = TowerRun(wa), TowerRun(wb)
    alone_a, alone_b = ra.encode(), rb.encode()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ra.out.fill_(float("nan"))
    rb.out.fill_(float("nan"))
    torch.cuda.synchronize()
    for _ in range(3):
        _encode(ra, sa)
        _encode(rb, sb)
    torch.cuda.synchronize()
    got_a = ra.out[: ra.plan.out_rows].cpu().numpy().astype(np.float64)
    got_b = rb.out[: rb.plan.out_rows].cpu().numpy().astype(np.float64)
    assert np.array_equal(got_a, alone_a) and np.array_equal(got_b, alone_b)
