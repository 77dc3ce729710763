"""The rocprofv3 summarizer behind profiles/ (CPU only): launch classes from kernel names in
dispatch order, and the derived columns of the counter and streaming tables on small
synthetic csv files."""

import csv

from multimodal_vlm_vision_amd import rocprof_summary as R


def gemm(epi, bm=128, occ=2, am=3):
    return f"void vitmi::(anonymous namespace)::gemm_kernel<{bm}, 256, 2, 2, {am}, {epi}, {occ}, false>(vitmi::GemmArgs)"


def attn(nw, part="false"):
    return (f"void vitmi::(anonymous namespace)::attn_kernel<80, {nw}, false, true, {part}>(vitmi::AttnArgs, "
            "vitmi::AttnWork const*, int, int const*)")


ROWNORM = "void vitmi::(anonymous namespace)::rownorm2_kernel<0, 10, 3, false>(vitmi::NormArgs)"
MERGE = "void vitmi::(anonymous namespace)::attn_merge_kernel<80, true>(vitmi::AttnArgs, vitmi::AttnMerge const*, int)"

# one forward of a 2-layer tower: normalise, patch embedding, two blocks (the second with
# key-split attention and its merge), merger
FORWARD = [
    ("void vitmi::(anonymous namespace)::vt_pad_zero_kernel(unsigned short*, int, int, int)", "vt_pad_zero"),
    ("void vitmi::(anonymous namespace)::normpatch_kernel<true>(vitmi::NormpatchArgs)", "normpatch"),
    (gemm(0, am=0), "gemm_patch_embed"),
    (ROWNORM, "rownorm"), (gemm(4), "gemm_qkv_rope"), (attn(4), "attention"), (attn(1), "attention_short"),
    (gemm(1), "gemm_proj_residual"), (ROWNORM, "rownorm"), (gemm(2), "gemm_fc1_gelu"),
    (gemm(1), "gemm_fc2_residual"),
    (ROWNORM, "rownorm"), (gemm(4), "gemm_qkv_rope"), (attn(4, "true"), "attention"), (MERGE, "attention_merge"),
    (gemm(1), "gemm_proj_residual"), (ROWNORM, "rownorm"), (gemm(3), "gemm_gateup_swiglu"),
    (gemm(1), "gemm_fc2_residual"),
    ("void vitmi::(anonymous namespace)::rownorm_kernel<0, 5, 3, false>(vitmi::NormArgs)", "rownorm"),
    (gemm(2), "gemm_merger_fc1_gelu"), (gemm(5), "gemm_merger_fc2"),
    ("__amd_rocclr_copyBuffer", "copy"),
]


def test_launch_classes_follow_the_forward():
    names = [n for n, _ in FORWARD]
    assert R.classify(names) == [c for _, c in FORWARD]
    # the class of a residual product depends on its position after qkv, not on its tile
    swapped = [gemm(4), gemm(1, bm=256, occ=1), gemm(2), gemm(1, bm=192, occ=1)]
    assert R.classify(swapped) == ["gemm_qkv_rope", "gemm_proj_residual", "gemm_fc1_gelu", "gemm_fc2_residual"]


def test_short_names():
    assert R.short_name(gemm(2)) == "gemm_kernel<128, 256, 2, 2, 3, 2, 2, false>"
    assert R.short_name(MERGE) == "attn_merge_kernel<80, true>"


def _write_counters(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_counter_table_fractions(tmp_path):
    """Two passes over one fc1 launch of 100 us at 2 GHz (200,000 cycles): the table's
    percentages are the counters over cycles x 1024 SIMDs, x 256 CUs, or over the cycles."""
    cyc = 200_000
    grbm = 8 * cyc                      # summed over the 8 XCDs
    t0, t1 = 1_000_000, 1_100_000       # ns
    k = gemm(2)
    p1, p2 = tmp_path / "p1", tmp_path / "p2"
    p1.mkdir()
    p2.mkdir()
    _write_counters(p1 / "p_counter_collection.csv", [
        (7, k, "GRBM_GUI_ACTIVE", grbm, t0, t1),
        (7, k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * 1024, t0, t1),
        (7, k, "SQ_LDS_IDX_ACTIVE", 0.25 * cyc * 256, t0, t1),
        (7, k, "SQ_LDS_BANK_CONFLICT", 0.05 * cyc * 256, t0, t1),
        (7, k, "TA_BUSY_avr", 0.6 * cyc, t0, t1),
    ])
    _write_counters(p2 / "p_counter_collection.csv", [
        (3, k, "GRBM_GUI_ACTIVE", grbm, t0, t1),
        (3, k, "TD_TD_BUSY_sum", 0.8 * cyc * 256, t0, t1),
        (3, k, "TCP_TCC_READ_REQ_sum", 1000.0, t0, t1),
        (3, k, "TCP_TCC_READ_REQ_LATENCY_sum", 250_000.0, t0, t1),
    ])
    out = tmp_path / "c.md"
    R.cmd_counters(str(out), "rocprofv3 ...", [str(p1), str(p2)])
    row = [l for l in out.read_text().splitlines() if l.startswith("| gemm_fc1_gelu |")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    # class, duration, clock, MFMA busy, VALU beside MFMA, LDS active, conflicts, TA, TD, L1
    # stall, L2 latency, read bytes per CU and cycle
    assert cells[1] == "100.0" and cells[2] == "2.00"
    assert cells[3] == "50%" and cells[4] == "--" and cells[5] == "25%" and cells[6] == "20%"
    assert cells[7] == "60%" and cells[8] == "80%" and cells[9] == "--"
    assert cells[10] == "250"
    assert cells[11] == f"{1000 * 128 / (cyc * 256):.1f}"


def test_kernel_digest_tracks_the_sources():
    d = R.kernel_sources_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert R.kernel_sources_digest() == d


def test_stream_table(tmp_path):
    """normpatch streaming summary: the launches with the largest grid, bandwidth from the
    algorithmic bytes, counter bytes scaled by the 512 MiB calibration copies."""
    np_name = "void vitmi::(anonymous namespace)::normpatch_kernel<true>(vitmi::NormpatchArgs)"
    cp_name = "__amd_rocclr_copyBuffer"
    trace = tmp_path / "trace"
    trace.mkdir()
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"]
    with open(trace / "p_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(cols)
        w.writerow([1, np_name, 4096, 0, 13_000])              # the forward's small launch: ignored
        w.writerow([2, np_name, 1 << 20, 20_000, 220_000])     # 200 us
        w.writerow([3, np_name, 1 << 20, 300_000, 520_000])    # 220 us
    alg = 48 * 1344 * 1344 * 3 + 48 * 96 * 96 * 1176 * 2

    def pmc(name, counter, kib_copy, kib_np):
        d = tmp_path / name
        d.mkdir()
        rows = [(i, cp_name, "Grid_Size", counter, kib_copy, 10 * i, 10 * i + 5) for i in range(3)]
        rows += [(9, np_name, "Grid_Size", counter, kib_np, 100, 200)]
        with open(d / "p_counter_collection.csv", "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
                        "Start_Timestamp", "End_Timestamp"])
            for r in rows:
                w.writerow([r[0], r[1], 1 << 20, r[3], r[4], r[5], r[6]])
        return str(d)

    f = pmc("fetch", "FETCH_SIZE", 262144, 150_000)   # factor 2
    wr = pmc("write", "WRITE_SIZE", 524288, 1_000_000)  # factor 1
    out = tmp_path / "s.md"
    R.cmd_stream(str(trace), f, wr, str(out), "rocprofv3 ...")
    row = [l for l in out.read_text().splitlines() if l.startswith("| 210.0 |")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "200.0" and cells[2] == "220.0"
    assert cells[3] == f"{alg / 210e-6 / 1e9:.0f}"
    assert cells[5] == f"{150_000 * 1024 * 2 / 1e6:.1f}" and cells[6] == f"{1_000_000 * 1024 / 1e6:.1f}"
