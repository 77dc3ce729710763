"""Vision-tower forward throughput on one MI355X.

Workload: the 8-image mixed-resolution batch (seeded sides 28 * U{8..48} px,
17,624 patches), Qwen2-VL-shaped 32-layer tower (hidden 1280, 16 heads of 80,
LayerNorm, GELU MLP 5120, 2D RoPE, per-image block-diagonal attention, 2x2
patch merger to 3584), bf16 MFMA with fp32 accumulation, random N(0, 0.02)
weights, uint8 pixels already in HBM.  One step = one whole forward (uint8
pixels -> normalise/patchify -> 32 blocks -> merger), replayed as one HIP
graph; K steps are timed between device synchronisations.

Also reported: a per-kernel breakdown from hipEvents around every launch
(one profiled eager forward per timed step), the dominant kernel's roofline
fraction, aggregate MFMA utilisation, the CPU oracle's throughput on a
bounded sample of the same batch (the three smallest images, full depth), and
a shape-bucketed graph captured for the batch replaying it and its first half
of items, against that half's own exact-shape graph, and the batch through
the vision-embedding cache (cold, warm, and the content-key pass alone), and
the device resize of the batch's images made off-grid.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-cpu]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "vision patches/sec (bf16 32-layer ViT, mixed-res batch) + MFMA util % of peak"
WORKLOAD = 3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(wl, items=None):
    """The CPU oracle (float32 NumPy, the precision it uses for the 1280-wide towers) on the
    headline batch -- every item, or the given subset -- timed around the forward only
    (inputs drawn beforehand), on this host's cores.  `cores` = the oracle's worker threads."""
    import numpy as np
    from oracle import vit_oracle
    sel = list(range(len(wl.items))) if items is None else list(items)
    n = sum(wl.items[i].n_patches for i in sel)
    threads = vit_oracle._threads()
    t0 = time.perf_counter()
    vit_oracle.forward_workload(wl, items=sel, dtype=np.float32)
    dt = time.perf_counter() - t0
    what = "the whole batch" if len(sel) == len(wl.items) else f"items {sel} of the batch"
    return {"value": n / dt, "unit": "patches/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what} ({n} patches), all {wl.cfg.layers} layers + merger, float32 NumPy "
                      f"(BLAS and a {threads}-thread pool), {dt:.1f} s"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_qwen2vl-8img-mixed-32L.md")


def kernel_sources_digest():
    """sha256 over the HIP kernel sources and the header they share (its layout helpers are
    kernel code): counter figures taken with other kernels are stale."""
    from multimodal_vlm_vision_amd.rocprof_summary import kernel_sources_digest as digest
    return digest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary (copy-calibrated), or None when absent or taken with different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None, None
    if data.get("kernel_sources_sha256_16") != kernel_sources_digest():
        return None, "stale: kernels changed since the counters were taken"
    row = data.get("per_launch", {}).get(kernel)
    if not row:
        return None, None
    return row["fetch_bytes"] + row["write_bytes"], os.path.relpath(TRAFFIC_FILE, ROOT)


def normpatch_stream(n_images=48, side=1344, reps=20):
    """normpatch alone on a >= 1 GB streaming batch (48 images of 1344 x 1344): the
    per-forward traffic of the bench batch (~52 MB) fits in the 256 MB last-level cache,
    so HBM bandwidth is measured on a batch several times larger than that cache.
    A zero-layer tower of width 64 keeps the rest of the forward negligible."""
    import dataclasses
    import numpy as np
    import torch
    from multimodal_vlm_vision_amd import VisionTower
    from workloads import make_weights, tower_config

    cfg = dataclasses.replace(tower_config(1), name="normpatch-stream", layers=0, mlp_dim=64, out_dim=64)
    tower = VisionTower(cfg)
    tower.load_weights(make_weights(99, cfg))
    tower.finalize()
    g = side // 14
    grid = np.array([[1, g, g]] * n_images, dtype=np.int32)
    plan = tower.plan(grid, np.ones(n_images, dtype=np.int32))
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    pixels = torch.randint(0, 256, (plan.pixel_bytes,), dtype=torch.uint8, device=dev, generator=gen)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(plan.out_rows, plan.out_cols, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    tower.encode(plan, pixels, ws, out, stream)
    tot_ms, by, n = 0.0, 0.0, 0
    for _ in range(reps):
        for k in tower.encode_profiled(plan, pixels, ws, out, stream):
            if k["name"] == "normpatch":
                tot_ms += k["total_ms"]
                by += k["bytes"]
                n += k["launches"]
    torch.cuda.synchronize()
    gbs = by / (tot_ms * 1e-3) / 1e9
    res = {"images": n_images, "side_px": side, "patches": int(grid[:, 1].sum() * g),
           "bytes_per_launch": by / n, "avg_us": tot_ms / n * 1e3, "gbs": gbs,
           "hbm_frac": gbs / PEAK_HBM_GBS}
    tower.close()
    return res


def pixels_upload(pixels_host, steps):
    """Host -> device copy of the batch's uint8 pixels from pinned memory, the step before the
    forward when frames arrive in host memory (reported beside the forward, never in it)."""
    import torch
    src = torch.from_numpy(pixels_host).pin_memory()
    dst = torch.empty(src.numel(), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        dst.copy_(src, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"bytes": int(src.numel()), "ms": ms, "gbs": src.numel() / (ms * 1e-3) / 1e9}


def resize_measure(wl, steps):
    """Device resize of the batch's images, each made off-grid by a seeded offset of up to 13
    pixels per side, back to the 28-pixel grid: one launch per image, all on one stream, timed
    with events; bytes = source read once + output written once (algorithmic)."""
    import numpy as np
    import torch
    from multimodal_vlm_vision_amd import resize_side, resize_u8

    g = np.random.default_rng(1234)

    def run(shapes):
        jobs = []
        for F, H, W in shapes:
            h, w = H + int(g.integers(1, 14)), W - int(g.integers(1, 14))
            src = torch.from_numpy(g.integers(0, 256, size=(F, h, w, 3), dtype=np.uint8)).cuda()
            dst = torch.empty(F, resize_side(h), resize_side(w), 3, dtype=torch.uint8, device="cuda")
            jobs.append((src, h, w, F, dst))
        moved = sum(s.numel() + d.numel() for s, _, _, _, d in jobs)

        def batch():
            for src, h, w, F, dst in jobs:
                resize_u8(src, h, w, F, dst)

        batch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            batch()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gbs = moved / (ms * 1e-3) / 1e9
        return {"images": len(jobs), "bytes": moved, "ms": ms, "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}

    res = run([it.frames.shape[:3] for it in wl.items])
    # a streaming batch far larger than the last-level cache: 48 images of about 1344 x 1344
    res["stream"] = run([(1, 1344, 1344)] * 48)
    return res


def cache_replay(tower, plan, pixels, ws, out, wl, steps, stream):
    """The batch through the vision-embedding cache: cold (every item encoded and inserted) and
    warm (every item served from the arena), plus the content-key pass alone.  Wall time per
    call; each call synchronises once on its keys."""
    import torch
    from multimodal_vlm_vision_amd import EmbeddingCache

    arena = torch.empty(plan.out_rows * plan.out_cols * 4 + (1 << 20), dtype=torch.uint8, device="cuda")

    def wall(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / n * 1e3

    cold = []
    for _ in range(2):
        cache = EmbeddingCache(tower, arena)
        cold.append(wall(lambda: tower.encode_cached(cache, plan, pixels, ws, out, stream), 1))
        cache.close()
    cache = EmbeddingCache(tower, arena)
    tower.encode_cached(cache, plan, pixels, ws, out, stream)
    warm_ms = wall(lambda: tower.encode_cached(cache, plan, pixels, ws, out, stream), steps)
    cache.close()
    keys_ms = wall(lambda: tower.pixel_keys(plan, pixels, ws, stream), steps)
    return {"items": len(wl.items), "cold_ms": min(cold), "warm_ms": warm_ms, "keys_ms": keys_ms,
            "pixel_bytes": plan.pixel_bytes, "key_gbs": plan.pixel_bytes / (keys_ms * 1e-3) / 1e9}


def bucket_replay(tower, plan, wl, steps, warmup, stream):
    """One bucketed graph captured for the batch (the capacity) replays the batch and a smaller
    batch (its first half of items) through vit_graph_launch_plan, against that smaller batch's
    own exact-shape graph: the cost of serving mixes from one capture."""
    import torch
    from workloads import pack_pixels

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps * 1e3

    sub_items = wl.items[:max(1, len(wl.items) // 2)]
    g = [it.grid_thw for it in sub_items]
    f = [it.n_frames for it in sub_items]
    sub = tower.plan(g, f)
    px_full = torch.from_numpy(pack_pixels(wl.items)).cuda()
    px_sub = torch.from_numpy(pack_pixels(sub_items)).cuda()
    bws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    bg = tower.capture_bucket(plan, bws)
    off = bg.pixels_ptr - bws.data_ptr()
    bws[off:off + px_full.numel()].copy_(px_full)
    full_ms = timed(lambda: bg.launch_plan(plan, stream))
    bws[off:off + px_sub.numel()].copy_(px_sub)
    sub_ms = timed(lambda: bg.launch_plan(sub, stream))
    bg.close()
    del bws
    sws = torch.empty(sub.ws_bytes, dtype=torch.uint8, device="cuda")
    sg = tower.capture(sub, sws)
    soff = sg.pixels_ptr - sws.data_ptr()
    sws[soff:soff + px_sub.numel()].copy_(px_sub)
    exact_ms = timed(lambda: sg.launch(stream))
    sg.close()
    return {"capacity_patches": plan.n_patches, "full_ms": full_ms, "subset_items": len(sub_items),
            "subset_patches": sub.n_patches, "subset_ms": sub_ms, "subset_exact_graph_ms": exact_ms,
            "subset_overhead_pct": 100.0 * (sub_ms / exact_ms - 1.0)}


def kernel_breakdown(tower, plan, pixels, ws, out, stream, steps):
    """Per-kernel-class totals from hipEvents around every launch (vit_encode_profiled) over
    `steps` eager forwards: {name: {launches, total_ms, flops, bytes, mfma_bound}}."""
    agg = {}
    for _ in range(steps):
        for k in tower.encode_profiled(plan, pixels, ws, out, stream):
            a = agg.setdefault(k["name"], {"launches": 0, "total_ms": 0.0, "flops": 0.0, "bytes": 0.0,
                                           "mfma_bound": k["mfma_bound"]})
            for f in ("launches", "total_ms", "flops", "bytes"):
                a[f] += k[f]
    return agg


def kernel_table(agg, steps):
    kern = {}
    tot_ms = sum(a["total_ms"] for a in agg.values())
    for name, a in sorted(agg.items(), key=lambda kv: -kv[1]["total_ms"]):
        avg_ms = a["total_ms"] / a["launches"]
        e = {"launches_per_step": a["launches"] // steps, "avg_us": avg_ms * 1e3,
             "share_pct": 100.0 * a["total_ms"] / tot_ms}
        if a["mfma_bound"]:
            e["tflops"] = a["flops"] / (a["total_ms"] * 1e-3) / 1e12
            e["mfma_pct"] = 100.0 * e["tflops"] / PEAK_BF16_TFLOPS
        else:
            e["gbs"] = a["bytes"] / (a["total_ms"] * 1e-3) / 1e9
            e["hbm_pct"] = 100.0 * e["gbs"] / PEAK_HBM_GBS
        kern[name] = e
    return kern


def roofline_of(agg, name):
    a = agg[name]
    per_launch_ms = a["total_ms"] / a["launches"]
    if a["mfma_bound"]:
        achieved = a["flops"] / a["launches"] / (per_launch_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None, "kernel": name,
                "avg_launch_us": per_launch_ms * 1e3}
    achieved = a["bytes"] / a["launches"] / (per_launch_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": name,
            "avg_launch_us": per_launch_ms * 1e3}


def measure_workload(index, steps, warmup, activations, stream):
    """Graph and eager throughput of one of the other workloads, with its per-kernel breakdown
    and the roofline fraction of its dominant kernel."""
    import torch
    from multimodal_vlm_vision_amd import VisionTower
    from workloads import make_workload, pack_pixels

    t0 = time.perf_counter()
    wl = make_workload(index)
    cfg = wl.cfg
    tower = VisionTower(cfg, activation_precision=activations)
    tower.load_weights(wl.weights)
    tower.finalize()
    plan = tower.plan(wl.grid_thw, wl.n_frames)
    pixels = torch.from_numpy(pack_pixels(wl.items)).cuda()
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(plan.out_rows, plan.out_cols, dtype=torch.float32, device="cuda")
    gws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    graph = tower.capture(plan, gws)
    off = graph.pixels_ptr - gws.data_ptr()
    gws[off:off + pixels.numel()].copy_(pixels)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps * 1e3

    graph_ms = timed(lambda: graph.launch(stream))
    eager_ms = timed(lambda: tower.encode(plan, pixels, ws, out, stream))
    graph.close()
    del gws
    agg = kernel_breakdown(tower, plan, pixels, ws, out, stream, steps)
    kern = kernel_table(agg, steps)
    dom = max(agg, key=lambda n: agg[n]["total_ms"])
    flops_step = sum(a["flops"] for a in agg.values()) / steps
    res = {"workload": cfg.name, "items": len(wl.items), "patches": wl.n_patches, "layers": cfg.layers,
           "graph_ms": graph_ms, "eager_ms": eager_ms, "graph_patches_per_s": wl.n_patches / (graph_ms * 1e-3),
           "eager_patches_per_s": wl.n_patches / (eager_ms * 1e-3),
           "mfma_util_pct": 100.0 * flops_step / (graph_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
           "algorithmic_tflop_per_step": flops_step / 1e12, "roofline": roofline_of(agg, dom),
           "kernels": kern}
    log(f"workload {cfg.name}: N={wl.n_patches}, graph {graph_ms:.3f} ms ({res['graph_patches_per_s']:,.0f} "
        f"patches/s), eager {eager_ms:.3f} ms, MFMA {res['mfma_util_pct']:.1f}% of peak "
        f"({time.perf_counter() - t0:.1f} s)")
    for name, e in kern.items():
        log(f"    {name:24s} {e['share_pct']:5.1f}%  avg {e['avg_us']:9.1f} us  " +
            (f"{e['tflops']:7.1f} TFLOP/s ({e['mfma_pct']:.1f}% MFMA)" if "tflops" in e
             else f"{e['gbs']:7.1f} GB/s ({e['hbm_pct']:.1f}% HBM)"))
    tower.close()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--workload", type=int, default=WORKLOAD)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 512 MiB device-to-device copy (3 times): the known-size kernel "
                         "that scales the HBM byte counters of a rocprofv3 --pmc run")
    ap.add_argument("--no-stream", action="store_true", help="skip the normpatch streaming measurement")
    ap.add_argument("--no-bucket", action="store_true", help="skip the shape-bucketed graph measurement")
    ap.add_argument("--no-cache", action="store_true", help="skip the embedding-cache measurement")
    ap.add_argument("--no-resize", action="store_true", help="skip the device-resize measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (tiny tower, 448 px tower, 16-frame video, Qwen2.5-shaped batch)")
    ap.add_argument("--cpu-items", default="all",
                    help="items of the batch the CPU oracle runs on: 'all' or a comma list of indices")
    ap.add_argument("--activations", default="f16", choices=["f16", "bf16f8", "bf16x2"],
                    help="form of the GEMM / attention activations: float16 (default), or bf16 compensated "
                         "by an e4m3 residual or by hi+lo bf16 pairs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the vision tower is not sharded "
              "across GPUs by this library", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from multimodal_vlm_vision_amd import VisionTower
    from workloads import make_workload, pack_pixels

    t0 = time.perf_counter()
    wl = make_workload(args.workload)
    cfg = wl.cfg
    log(f"workload {cfg.name}: {len(wl.items)} items, N={wl.n_patches} patches, "
        f"grids={[it.grid_thw for it in wl.items]} ({time.perf_counter() - t0:.1f} s to draw)")
    dev = torch.device("cuda:0")
    tower = VisionTower(cfg, activation_precision=args.activations)
    tower.load_weights(wl.weights)
    tower.finalize()
    plan = tower.plan(wl.grid_thw, wl.n_frames)
    pixels = torch.from_numpy(pack_pixels(wl.items)).to(dev)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(plan.out_rows, plan.out_cols, dtype=torch.float32, device=dev)
    log(f"weights uploaded, workspace {plan.ws_bytes / 2**20:.0f} MiB ({time.perf_counter() - t0:.1f} s)")

    # ---- graph: the whole forward, normalisation included, replayed
    gws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=dev)
    graph = tower.capture(plan, gws)
    off = graph.pixels_ptr - gws.data_ptr()
    gws[off:off + pixels.numel()].copy_(pixels)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        graph.launch(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        graph.launch(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t1
    ms_step = dt / args.steps * 1e3
    value = wl.n_patches / (dt / args.steps)
    log(f"graph: {ms_step:.3f} ms/step, {value:,.0f} patches/s")

    # ---- eager (no events) for reference
    for _ in range(2):
        tower.encode(plan, pixels, ws, out, stream)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        tower.encode(plan, pixels, ws, out, stream)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t2) / args.steps * 1e3

    # ---- per-kernel breakdown: hipEvents around every launch, same stream
    agg = kernel_breakdown(tower, plan, pixels, ws, out, stream, args.steps)
    kern = kernel_table(agg, args.steps)
    for name, e in kern.items():
        log(f"  {name:24s} {e['share_pct']:5.1f}%  avg {e['avg_us']:9.1f} us  " +
            (f"{e['tflops']:7.1f} TFLOP/s ({e['mfma_pct']:.1f}% MFMA)" if "tflops" in e
             else f"{e['gbs']:7.1f} GB/s ({e['hbm_pct']:.1f}% HBM)"))
    dom = max(agg, key=lambda n: agg[n]["total_ms"])
    roof = roofline_of(agg, dom)
    flops_step = sum(a["flops"] for a in agg.values()) / args.steps
    mfma_util = 100.0 * flops_step / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)

    line = {
        "metric": METRIC, "value": value, "unit": "patches/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16" if args.activations == "f16" else "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "items": len(wl.items), "patches": wl.n_patches,
                   "layers": cfg.layers, "hidden": cfg.hidden, "heads": cfg.heads, "mlp": cfg.mlp_dim,
                   "out_dim": cfg.out_dim, "mode": "hipgraph", "parallelism": "single-gpu",
                   "weights": "bf16", "activations": args.activations},
        "mfma_util_pct": mfma_util,
        "algorithmic_tflop_per_step": flops_step / 1e12,
        "eager_ms_per_step": eager_ms,
        "roofline": roof,
        "kernels": kern,
    }
    graph.close()
    roof["traffic"], roof["traffic_source"] = measured_traffic(dom)
    line["pixels_h2d"] = pixels_upload(pack_pixels(wl.items), args.steps)
    log(f"pixel upload (pinned host -> device): {line['pixels_h2d']['bytes'] / 1e6:.1f} MB, "
        f"{line['pixels_h2d']['ms']:.3f} ms, {line['pixels_h2d']['gbs']:.1f} GB/s")
    if not args.no_resize:
        line["resize"] = resize_measure(wl, args.steps)
        r = line["resize"]
        for tag, q in (("batch", r), ("stream", r["stream"])):
            log(f"device resize ({tag}): {q['images']} off-grid images, {q['bytes'] / 1e6:.1f} MB moved, "
                f"{q['ms']:.3f} ms, {q['gbs']:.0f} GB/s ({100 * q['hbm_frac']:.1f}% of HBM peak)")
    if not args.no_cache:
        line["embedding_cache"] = cache_replay(tower, plan, pixels, ws, out, wl, args.steps, stream)
        c = line["embedding_cache"]
        log(f"embedding cache: cold {c['cold_ms']:.3f} ms, warm (all {c['items']} items cached) "
            f"{c['warm_ms']:.3f} ms; content keys alone {c['keys_ms']:.3f} ms "
            f"({c['key_gbs']:.0f} GB/s of pixels)")
    if not args.no_bucket:
        line["bucket"] = bucket_replay(tower, plan, wl, args.steps, args.warmup, stream)
        b = line["bucket"]
        log(f"bucketed graph (capacity {b['capacity_patches']} patches): full batch {b['full_ms']:.3f} ms; "
            f"{b['subset_patches']}-patch batch {b['subset_ms']:.3f} ms vs {b['subset_exact_graph_ms']:.3f} ms "
            f"in its own graph")
    if not args.no_stream:
        log("normpatch streaming measurement ...")
        line["normpatch_stream"] = normpatch_stream()
        ns = line["normpatch_stream"]
        log(f"normpatch stream: {ns['patches']} patches, {ns['bytes_per_launch'] / 1e9:.2f} GB/launch, "
            f"{ns['avg_us']:.1f} us, {ns['gbs']:.0f} GB/s ({100 * ns['hbm_frac']:.1f}% of HBM peak)")
    if args.calibrate_copy:
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 x 512 MiB device-to-device")
    if not args.no_configs:
        del ws, gws
        tower.close()
        torch.cuda.empty_cache()
        line["workloads"] = {}
        for idx in (1, 2, 4, 5):
            line["workloads"][f"w{idx}"] = measure_workload(idx, args.steps, args.warmup, args.activations,
                                                            stream)
            torch.cuda.empty_cache()
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        items = None if args.cpu_items == "all" else [int(i) for i in args.cpu_items.split(",")]
        line["cpu_baseline"] = cpu_baseline(wl, items)
        log(f"CPU oracle: {line['cpu_baseline']['value']:.1f} patches/s on {line['cpu_baseline']['cores']} threads")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
