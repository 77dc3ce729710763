"""Summaries of rocprofv3 runs of bench.py, as the short markdown files kept under profiles/.

    python -m multimodal_vlm_vision_amd.rocprof_summary trace   <dir> <out.md> "<command>" [workload index]
    python -m multimodal_vlm_vision_amd.rocprof_summary traffic <fetch dir> <write dir> <out.md> "<commands>"
    python -m multimodal_vlm_vision_amd.rocprof_summary mfma    <dir> <out.md> "<command>"
    python -m multimodal_vlm_vision_amd.rocprof_summary counters <out.md> "<command>" <dir> [<dir> ...]
    python -m multimodal_vlm_vision_amd.rocprof_summary stream  <trace dir> <fetch dir> <write dir> <out.md> "<commands>"

<dir> is a rocprofv3 output directory (``--output-format csv``); the csv files are found
recursively.  Every dispatch is assigned to a launch class of the forward from its kernel's
template arguments and its position in the forward (the out-projection and fc2 share one
kernel: the first residual product after a qkv launch is the out-projection); the class names
are the ones bench.py and vit_encode_profiled use.  Algorithmic figures are those of the
workload given (default: the 8-image headline batch, workloads.make_workload(3)).
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

EPI_NAMES = {0: "gemm_patch_embed", 2: "gemm_fc1_gelu", 3: "gemm_gateup_swiglu", 4: "gemm_qkv_rope",
             5: "gemm_merger_fc2"}


def _rows(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    low = {k.lower(): k for k in row}
    for n in names:
        if n.lower() in low:
            return row[low[n.lower()]]
    raise KeyError(names)


def short_name(name: str) -> str:
    """`gemm_kernel<128, 256, 2, 2, 3, 1, 2, false>` from a demangled kernel name."""
    m = re.search(r"(\w+_kernel\w*)<([^>]*)>", name)
    if m:
        return f"{m.group(1)}<{m.group(2)}>"
    m = re.search(r"(\w+_kernel\w*)", name)
    return m.group(1) if m else name.split("(")[0][-60:]


def _targs(name: str):
    m = re.search(r"<([^>]*)>", name)
    return [a.strip() for a in m.group(1).split(",")] if m else []


def classify(names):
    """Launch class of every dispatch, given the kernel names in dispatch order."""
    classes = []
    gemm_epi = [None] * len(names)
    for i, nm in enumerate(names):
        if "gemm_kernel" in nm:
            a = _targs(nm)
            gemm_epi[i] = int(a[5]) if len(a) >= 6 else None
    since_qkv = 0
    for i, nm in enumerate(names):
        if "vt_pad_zero" in nm:
            c = "vt_pad_zero"
        elif "normpatch_kernel" in nm:
            c = "normpatch"
        elif "normrows_kernel" in nm:
            c = "normrows_u8"
        elif "rownorm" in nm:
            c = "rownorm"
        elif "attn_merge_kernel" in nm:
            c = "attention_merge"
        elif "attn_kernel" in nm:
            a = _targs(nm)
            c = "attention" if len(a) >= 2 and a[1] == "4" else "attention_short"
        elif "gemm_kernel" in nm:
            e = gemm_epi[i]
            if e == 4:
                since_qkv = 0
                c = "gemm_qkv_rope"
            elif e == 1:
                since_qkv += 1
                c = "gemm_proj_residual" if since_qkv == 1 else "gemm_fc2_residual"
            elif e == 2:
                nxt = next((gemm_epi[j] for j in range(i + 1, len(names)) if gemm_epi[j] is not None), None)
                c = "gemm_merger_fc1_gelu" if nxt == 5 else "gemm_fc1_gelu"
            else:
                c = EPI_NAMES.get(e, "gemm_other")
        elif "copy" in nm.lower():
            c = "copy"
        else:
            c = "other"
        classes.append(c)
    return classes


def _dispatches(rows):
    """[(dispatch id, name, start, end, row)] in dispatch order."""
    out = []
    for r in rows:
        did = int(_col(r, "Dispatch_Id", "Dispatch_ID"))
        out.append((did, _col(r, "Kernel_Name"), int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp")), r))
    out.sort(key=lambda x: (x[2], x[0]))
    return out


def _window_lengths(items, window_units):
    """Patch counts of the attention windows: per frame, square windows of window_units x
    window_units merge units tiled from the top-left, truncated at the edges."""
    out = []
    for it in items:
        t, h, w = it.grid_thw
        uh, uw = h // 2, w // 2
        for _ in range(t):
            for wy in range(0, uh, window_units):
                for wx in range(0, uw, window_units):
                    out.append(4 * min(window_units, uh - wy) * min(window_units, uw - wx))
    return out


def headline_algorithmic(index: int = 3):
    """Algorithmic MFMA FLOPs and HBM bytes per launch of each class on workload `index`
    (3, the 8-image headline batch, by default).  Attention classes average over their
    launches: 'attention' runs the long units (segments above 128 patches) of the item-segment
    layers, 'attention_short' the short ones and, in windowed towers, the window layers."""
    sys.path.insert(0, ROOT)
    from workloads import make_workload
    wl = make_workload(index, with_weights=False)
    c = wl.cfg
    N = wl.n_patches
    d, mlp, out, K = c.hidden, c.mlp_dim, c.out_dim, 1176
    U = N // 4
    segs = wl.seg_lengths
    sq = float(sum(n * n for n in segs))
    sq_long = float(sum(n * n for n in segs if n > 128))
    sq_short = float(sum(n * n for n in segs if n <= 128))
    if c.window_px:
        n_full = len(c.full_attn_layers)
        n_win = c.layers - n_full
        sq_win = float(sum(n * n for n in _window_lengths(wl.items, c.window_px // 28)))
        short_launches = n_win + (n_full if sq_short else 0)
        attn_short = 4.0 * d * (n_win * sq_win + n_full * sq_short) / max(short_launches, 1)
    else:
        attn_short = 4.0 * d * sq_short
    b = 2   # float16 / bfloat16 operands
    mlp_mult = 2 if c.mlp_kind == "swiglu" else 1
    flops = {"gemm_patch_embed": 2.0 * N * d * K, "gemm_qkv_rope": 2.0 * N * 3 * d * d,
             "attention": 4.0 * d * sq_long, "attention_short": attn_short,
             "gemm_proj_residual": 2.0 * N * d * d,
             "gemm_fc1_gelu": 2.0 * N * d * mlp, "gemm_gateup_swiglu": 2.0 * N * d * mlp * mlp_mult,
             "gemm_fc2_residual": 2.0 * N * mlp * d,
             "gemm_merger_fc1_gelu": 2.0 * U * 16 * d * d, "gemm_merger_fc2": 2.0 * U * 4 * d * out}
    px = sum(it.frames.size for it in wl.items)
    # bytes: every operand read once, every output written once (residual products read and
    # write the fp32 stream)
    byt = {"normpatch": px + N * K * 2, "rownorm": N * d * 4 + N * d * b,
           "gemm_patch_embed": N * K * 2 + d * K * 2 + N * d * 4,
           "gemm_qkv_rope": N * d * b + 3 * d * d * b + 3 * N * d * b,
           "attention": 4 * N * d * b,
           "gemm_proj_residual": N * d * b + d * d * b + 2 * N * d * 4,
           "gemm_fc1_gelu": N * d * b + mlp * d * b + N * mlp * b,
           "gemm_fc2_residual": N * mlp * b + d * mlp * b + 2 * N * d * 4,
           "gemm_merger_fc1_gelu": U * 4 * d * b + 16 * d * d * b + U * 4 * d * b,
           "gemm_merger_fc2": U * 4 * d * b + out * 4 * d * b + U * out * 4}
    return wl, flops, byt, sq


def kernel_sources_digest() -> str:
    """sha256 (16 hex digits) of the HIP kernel sources and their shared header, as bench.py computes it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "multimodal_vlm_vision_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cmd_trace(directory, out_md, command, index=3):
    disp = _dispatches(_rows(directory, "kernel_trace.csv"))
    classes = classify([d[1] for d in disp])
    by_name = defaultdict(list)
    by_class = defaultdict(list)
    cls_of_name = defaultdict(set)
    for (did, nm, s, e, _), c in zip(disp, classes):
        by_name[short_name(nm)].append((e - s) / 1e3)
        by_class[c].append((e - s) / 1e3)
        cls_of_name[short_name(nm)].add(c)
    total = sum(sum(v) for v in by_name.values())
    wl, flops, _, _ = headline_algorithmic(index)
    lines = [f"# rocprofv3 kernel statistics -- vision tower forward, {wl.cfg.name}", "",
             f"Workload: {wl.cfg.name} (N = {wl.n_patches} patches, hidden {wl.cfg.hidden}, {wl.cfg.heads} heads of "
             f"{wl.cfg.head_dim}, MLP {wl.cfg.mlp_dim}, out {wl.cfg.out_dim}), float16 activations (bf16 patch "
             "embedding), whole forward replayed as a HIP graph plus eager and profiled eager forwards.", "",
             "Command (from the repository root on an MI355X machine; <out> is any output directory):", "", "```", command, "```", "",
             "Per kernel (durations from the kernel trace):", "",
             "| Kernel | Launch class | Calls | Avg (µs) | Min (µs) | Max (µs) | % time |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for nm, v in sorted(by_name.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{nm}` | {', '.join(sorted(cls_of_name[nm]))} | {len(v)} | {sum(v) / len(v):.1f} | "
                     f"{min(v):.1f} | {max(v):.1f} | {100 * sum(v) / total:.2f} |")
    lines += ["", "Per launch class (the classes of bench.py's kernel table; MFMA classes against the "
              "2.5 PFLOP/s dense peak):", "",
              "| Launch class | Launches | Avg (µs) | Algorithmic GFLOP per launch | TFLOP/s | Fraction of peak |",
              "|---|---:|---:|---:|---:|---:|"]
    for c, v in sorted(by_class.items(), key=lambda kv: -sum(kv[1])):
        avg = sum(v) / len(v)
        if c in flops:
            tf = flops[c] / (avg * 1e-6) / 1e12
            lines.append(f"| {c} | {len(v)} | {avg:.1f} | {flops[c] / 1e9:.1f} | {tf:.1f} | {tf / 2500:.3f} |")
        else:
            lines.append(f"| {c} | {len(v)} | {avg:.1f} | -- | -- | -- |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _counter_rows(directory, counter):
    rows = [r for r in _rows(directory, "counter_collection.csv") if _col(r, "Counter_Name") == counter]
    out = []
    for r in rows:
        did = int(_col(r, "Dispatch_Id", "Dispatch_ID"))
        out.append((did, _col(r, "Kernel_Name"), float(_col(r, "Counter_Value")),
                    int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp"))))
    out.sort(key=lambda x: (x[0], x[3]))
    return out


def _per_class(rows):
    classes = classify([r[1] for r in rows])
    acc = defaultdict(list)
    for r, c in zip(rows, classes):
        acc[c].append(r)
    return acc


def cmd_traffic(fetch_dir, write_dir, out_md, command):
    f_cls = _per_class(_counter_rows(fetch_dir, "FETCH_SIZE"))
    w_cls = _per_class(_counter_rows(write_dir, "WRITE_SIZE"))
    copy_bytes = 512 << 20

    def calib(cls, want):
        # the calibration copies are the last three copy dispatches (bench.py --calibrate-copy runs
        # them after every forward); earlier copies are host uploads
        cp = sorted(cls.get("copy", []), key=lambda r: (r[3], r[0]))[-3:]
        if len(cp) < 3:
            raise RuntimeError("no calibration copies found (run bench.py with --calibrate-copy)")
        kib = sorted(r[2] for r in cp)[1]
        return want / (kib * 1024.0), kib

    f_fac, f_kib = calib(f_cls, copy_bytes)
    w_fac, w_kib = calib(w_cls, copy_bytes)
    wl, _, byt, _ = headline_algorithmic()
    per_launch = {}
    lines = [f"# HBM traffic per launch -- vision tower forward, {wl.cfg.name}", "",
             "Two counter passes over the bench, each with a 512 MiB device-to-device copy (3 times, "
             "`--calibrate-copy`) as the known-size reference.  Commands (from the repository root on an MI355X machine; <out> is any output directory):",
             "", "```", command, "```", "",
             f"Calibration: the 512 MiB copy reads as FETCH_SIZE {f_kib:.0f} KiB (factor {f_fac:.4f}) and WRITE_SIZE "
             f"{w_kib:.0f} KiB (factor {w_fac:.4f}); every figure below is the counter's KiB per dispatch x 1024 x its "
             "factor, averaged over the class's dispatches.  FETCH_SIZE counts L2 misses, which the 256 MB "
             "last-level cache may serve; it is an upper bound on HBM reads.", "",
             "| Launch class | Fetched (MB) | Written (MB) | Total (MB) | Algorithmic read + write (MB) | Ratio |",
             "|---|---:|---:|---:|---:|---:|"]
    order = ["normpatch", "gemm_patch_embed", "rownorm", "gemm_qkv_rope", "attention", "gemm_proj_residual",
             "gemm_fc1_gelu", "gemm_fc2_residual", "gemm_merger_fc1_gelu", "gemm_merger_fc2"]
    for c in order:
        if c not in f_cls or c not in w_cls:
            continue
        fb = sum(r[2] for r in f_cls[c]) / len(f_cls[c]) * 1024.0 * f_fac
        wb = sum(r[2] for r in w_cls[c]) / len(w_cls[c]) * 1024.0 * w_fac
        per_launch[c] = {"fetch_bytes": int(fb), "write_bytes": int(wb)}
        alg = byt.get(c)
        lines.append(f"| {c} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | "
                     f"{alg / 1e6:.1f} | {(fb + wb) / alg:.2f} |" if alg else
                     f"| {c} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | -- | -- |")
    data = {"kernel_sources_sha256_16": kernel_sources_digest(), "calibration_factors": [f_fac, w_fac],
            "per_launch": per_launch}
    lines += ["", "Machine-readable figures (bytes per launch; `bench.py` reports `roofline.traffic` from this "
              "block only while the HIP kernel sources and their shared header hash to the digest below):", "",
              "```json", json.dumps(data, indent=1), "```"]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def cmd_mfma(directory, out_md, command):
    names = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
             "GRBM_GUI_ACTIVE"]
    rows = _rows(directory, "counter_collection.csv")
    per = defaultdict(dict)
    meta = {}
    for r in rows:
        did = int(_col(r, "Dispatch_Id", "Dispatch_ID"))
        per[did][_col(r, "Counter_Name")] = float(_col(r, "Counter_Value"))
        meta[did] = (_col(r, "Kernel_Name"), int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp")))
    dids = sorted(meta, key=lambda d: (meta[d][1], d))
    classes = classify([meta[d][0] for d in dids])
    acc = defaultdict(list)
    for d, c in zip(dids, classes):
        acc[c].append(d)
    wl, flops, _, _ = headline_algorithmic()
    lines = [f"# MFMA hardware counters per launch class -- vision tower forward, {wl.cfg.name}", "",
             "One counter pass over the bench's forwards.  Command (from the repository root on an MI355X machine; <out> is any output directory):", "",
             "```", command, "```", "",
             "GRBM_GUI_ACTIVE reads as the sum over the 8 XCDs, so the clock column is GRBM_GUI_ACTIVE / 8 / duration "
             "and MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs) / (GRBM_GUI_ACTIVE / 8 x 1024).  "
             "Durations are those of the profiled (serialised) dispatches.  Executed MFMA FLOPs = "
             "SQ_INSTS_VALU_MFMA_MOPS_F16 (resp. _BF16) x 512 (the counters' unit); algorithmic FLOPs count each "
             "product once (2 per multiply-add, unpadded shapes; attention 4 * hidden * sum of squared segment "
             "lengths).", "",
             "| Launch class | Launches sampled | Duration (us) | Clock (GHz) | MFMA busy (%) | Executed f16 MFMA "
             "GFLOP per launch | Executed bf16 MFMA GFLOP per launch | Algorithmic GFLOP | Executed / algorithmic |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for c in ["gemm_patch_embed", "gemm_qkv_rope", "attention", "gemm_proj_residual", "gemm_fc1_gelu",
              "gemm_fc2_residual", "gemm_merger_fc1_gelu", "gemm_merger_fc2"]:
        ds = acc.get(c, [])
        if not ds:
            continue
        dur = sum(meta[d][2] - meta[d][1] for d in ds) / len(ds)
        g = sum(per[d].get(names[3], 0.0) for d in ds) / len(ds)
        busy = sum(per[d].get(names[0], 0.0) for d in ds) / len(ds)
        f16 = sum(per[d].get(names[1], 0.0) for d in ds) / len(ds) * 512
        b16 = sum(per[d].get(names[2], 0.0) for d in ds) / len(ds) * 512
        clock = g / 8 / dur if dur else 0.0
        mfma = 100 * busy / (g / 8 * 1024) if g else 0.0
        alg = flops[c]
        lines.append(f"| {c} | {len(ds)} | {dur / 1e3:.1f} | {clock:.2f} | {mfma:.1f} | {f16 / 1e9:.1f} | "
                     f"{b16 / 1e9:.1f} | {alg / 1e9:.1f} | {(f16 + b16) / alg:.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


# (counter, divisor kind, column title): "simd" divides by the cycles x 1024 SIMDs, "cu" by the
# cycles x 256 CUs, "cyc" by the cycles (an average over instances), "lds" by SQ_LDS_IDX_ACTIVE
_PATH_COLUMNS = [
    ("SQ_VALU_MFMA_BUSY_CYCLES", "simd", "MFMA busy"),
    ("SQ_VALU_MFMA_COEXEC_CYCLES", "simd", "VALU beside MFMA"),
    ("SQ_LDS_IDX_ACTIVE", "cu", "LDS active"),
    ("SQ_LDS_BANK_CONFLICT", "lds", "LDS bank conflicts (of LDS active)"),
    ("TA_BUSY_avr", "cyc", "TA busy"),
    ("TD_TD_BUSY_sum", "cu", "TD busy"),
    ("TCP_PENDING_STALL_CYCLES_sum", "cu", "L1 stalled on pending misses"),
]


def cmd_counters(out_md, command, dirs):
    """Memory-path and issue counters per launch class, from one or more counter passes (each
    pass carrying GRBM_GUI_ACTIVE for its clock), as fractions of the kernel's cycles."""
    per = defaultdict(dict)      # (pass, dispatch) -> counter -> value
    meta = {}
    order = []
    for i, d in enumerate(dirs):
        rows = _rows(d, "counter_collection.csv")
        m = {}
        for r in rows:
            did = int(_col(r, "Dispatch_Id", "Dispatch_ID"))
            per[(i, did)][_col(r, "Counter_Name")] = float(_col(r, "Counter_Value"))
            m[did] = (_col(r, "Kernel_Name"), int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp")))
        dids = sorted(m, key=lambda x: (m[x][1], x))
        for did, c in zip(dids, classify([m[x][0] for x in dids])):
            meta[(i, did)] = (c, m[did][2] - m[did][1])
            order.append((i, did))
    # (the ~23 us row norm is left out: for launches that short GRBM_GUI_ACTIVE also counts the
    # dispatch around the kernel and reads above the clock)
    classes = ["gemm_qkv_rope", "attention", "gemm_proj_residual", "gemm_fc1_gelu", "gemm_fc2_residual"]

    def avg(c, name):
        vals, cyc, dur = [], [], []
        for key in order:
            if meta[key][0] != c or name not in per[key]:
                continue
            vals.append(per[key][name])
            cyc.append(per[key].get("GRBM_GUI_ACTIVE", 0.0) / 8)
            dur.append(meta[key][1])
        if not vals:
            return None
        return sum(vals) / len(vals), sum(cyc) / len(cyc), sum(dur) / len(dur)

    head = ["Launch class", "Duration (us)", "Clock (GHz)"] + [t for _, _, t in _PATH_COLUMNS] + \
           ["L2 read latency (cycles)", "L1 <- L2 read bytes per CU and cycle"]
    lines = ["# Issue and memory-path counters per launch class -- vision tower forward, qwen2vl-8img-mixed-32L", "",
             "Counter passes over the bench's forwards, one rocprofv3 run per pass "
             f"(kernel sources digest {kernel_sources_digest()}).  Commands (from the repository root on an MI355X machine; <out> is any output directory; "
             "<counters> is each pass's list below):", "", "```", command, "```", ""]
    for i, d in enumerate(dirs):
        names = sorted({n for k, v in per.items() if k[0] == i for n in v})
        lines.append(f"* pass {i + 1}: {' '.join(names)}")
    lines += ["", "Cycles are GRBM_GUI_ACTIVE / 8 (it reads as the sum over the 8 XCDs).  MFMA busy and VALU "
              "beside MFMA are per SIMD (1024 SIMDs), LDS active, TD busy and the L1 stall per CU (256), TA busy "
              "is already an average over the TA instances; the L2 read latency is TCP_TCC_READ_REQ_LATENCY_sum "
              "/ TCP_TCC_READ_REQ_sum, and the read bytes count 128 bytes per L1 -> L2 read request.", "",
              "| " + " | ".join(head) + " |", "|---|" + "---:|" * (len(head) - 1)]
    for c in classes:
        g = avg(c, "GRBM_GUI_ACTIVE")
        if g is None:
            continue
        _, cyc, dur = g
        cells = [c, f"{dur / 1e3:.1f}", f"{cyc / dur:.2f}"]
        for name, kind, _ in _PATH_COLUMNS:
            a = avg(c, name)
            if a is None:
                cells.append("--")
                continue
            v, cy, _ = a
            if kind == "lds":
                b = avg(c, "SQ_LDS_IDX_ACTIVE")
                cells.append(f"{100 * v / b[0]:.0f}%" if b and b[0] else "--")
            else:
                div = {"simd": cy * 1024, "cu": cy * 256, "cyc": cy}[kind]
                cells.append(f"{100 * v / div:.0f}%" if div else "--")
        lat, req = avg(c, "TCP_TCC_READ_REQ_LATENCY_sum"), avg(c, "TCP_TCC_READ_REQ_sum")
        cells.append(f"{lat[0] / req[0]:.0f}" if lat and req and req[0] else "--")
        cells.append(f"{req[0] * 128 / (req[1] * 256):.1f}" if req and req[1] else "--")
        lines.append("| " + " | ".join(cells) + " |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def cmd_stream(trace_dir, fetch_dir, write_dir, out_md, command, n_images=48, side=1344):
    """normpatch on bench.py's streaming batch (n_images images of side x side pixels, one
    frame each): the launches with the largest grid among the normpatch dispatches.  Achieved
    bandwidth = algorithmic bytes (the uint8 pixels read once, the bf16 patch rows written
    once) / average duration; traffic from FETCH_SIZE / WRITE_SIZE scaled by the 512 MiB
    calibration copies."""
    g = side // 14
    n_patch = n_images * g * g
    alg_read = n_images * side * side * 3
    alg_write = n_patch * 1176 * 2

    def stream_rows(rows, name_col="Kernel_Name"):
        np_rows = [r for r in rows if "normpatch_kernel" in _col(r, name_col)]
        if not np_rows:
            raise RuntimeError("no normpatch dispatches")
        big = max(int(_col(r, "Grid_Size", "Grid_Size_X")) for r in np_rows)
        return [r for r in np_rows if int(_col(r, "Grid_Size", "Grid_Size_X")) == big], big

    tr, grid = stream_rows(_rows(trace_dir, "kernel_trace.csv"))
    durs = sorted(int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp")) for r in tr)
    avg = sum(durs) / len(durs)
    copy_bytes = 512 << 20

    def counter_bytes(directory, counter):
        rows = [r for r in _rows(directory, "counter_collection.csv") if _col(r, "Counter_Name") == counter]
        cp = sorted((r for r in rows if "copy" in _col(r, "Kernel_Name").lower()),
                    key=lambda r: (int(_col(r, "Start_Timestamp")), int(_col(r, "Dispatch_Id", "Dispatch_ID"))))[-3:]
        if len(cp) < 3:
            raise RuntimeError("no calibration copies found (run bench.py with --calibrate-copy)")
        kib = sorted(float(_col(r, "Counter_Value")) for r in cp)[1]
        fac = copy_bytes / (kib * 1024.0)
        sr, _ = stream_rows(rows)
        return sum(float(_col(r, "Counter_Value")) for r in sr) / len(sr) * 1024.0 * fac, fac, len(sr)

    fb, ffac, nf = counter_bytes(fetch_dir, "FETCH_SIZE")
    wb, wfac, nw = counter_bytes(write_dir, "WRITE_SIZE")
    alg = alg_read + alg_write
    gbs = alg / (avg * 1e-9) / 1e9
    lines = [f"# normpatch on a streaming batch -- {n_images} images of {side} x {side} pixels", "",
             f"The uint8 -> normalised bf16 patch-row kernel alone on bench.py's streaming batch ({n_patch} image "
             f"patches, {alg / 1e9:.2f} GB of algorithmic traffic per launch, several times the 256 MB last-level "
             "cache), inside the bench's normpatch_stream measurement (a zero-layer tower).  Commands (from the "
             "repository root on an MI355X machine; <out> is any output directory):", "", "```", command, "```", "",
             f"Launches of the streaming batch: the {len(tr)} normpatch dispatches with the largest grid "
             f"({grid} work-items) in the trace, {nf} and {nw} in the counter passes.  Algorithmic bytes per "
             f"launch: {alg_read / 1e6:.1f} MB of pixels read (an image's one frame serves both temporal "
             f"slots) + {alg_write / 1e6:.1f} MB of bf16 rows written (588 + 2352 bytes per image patch).", "",
             "| Avg (us) | Min (us) | Max (us) | Achieved (GB/s) | Fraction of 8 TB/s | Fetched (MB) | Written (MB) "
             "| Counter bytes / algorithmic |",
             "|---:|---:|---:|---:|---:|---:|---:|---:|",
             f"| {avg / 1e3:.1f} | {durs[0] / 1e3:.1f} | {durs[-1] / 1e3:.1f} | {gbs:.0f} | {gbs / 8000:.3f} | "
             f"{fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / alg:.3f} |", "",
             f"Counter calibration: FETCH_SIZE factor {ffac:.4f}, WRITE_SIZE factor {wfac:.4f} (512 MiB copy).  "
             f"Kernel sources digest {kernel_sources_digest()}."]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main(argv):
    if len(argv) >= 4 and argv[0] == "trace":
        cmd_trace(argv[1], argv[2], argv[3], int(argv[4]) if len(argv) >= 5 else 3)
    elif len(argv) >= 5 and argv[0] == "traffic":
        cmd_traffic(argv[1], argv[2], argv[3], argv[4])
    elif len(argv) >= 4 and argv[0] == "mfma":
        cmd_mfma(argv[1], argv[2], argv[3])
    elif len(argv) >= 4 and argv[0] == "counters":
        cmd_counters(argv[1], argv[2], argv[3:])
    elif len(argv) >= 6 and argv[0] == "stream":
        cmd_stream(argv[1], argv[2], argv[3], argv[4], argv[5])
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
