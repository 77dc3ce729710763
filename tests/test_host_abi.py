"""CPU tests of the C ABI's host side: the library loads and exports every
symbol the header declares; configuration, weight and batch validation fail
with the documented status before anything is enqueued; the planner's sizes,
row order and window permutation agree with index sets derived independently
(from the oracle's window partition); the header compiles as C99 and a C program linked
with the library runs the host-side calls.  No GPU call is made."""

import ctypes

import numpy as np
import pytest

from multimodal_vlm_vision_amd import binding as B
from oracle import vit_oracle as O
from workloads import TowerConfig, tower_config


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_library_exports_every_header_symbol(lib):
    names = B.header_symbols()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B._SIGS), "binding signatures must cover the header exactly"


def _status(fn):
    try:
        fn()
    except B.VitError as e:
        return e.status
    return B.VIT_OK


def test_config_validation(lib):
    import dataclasses
    cfg = tower_config(2)
    assert _status(lambda: B.VisionTower(cfg, lib)) == B.VIT_OK
    bad = [dataclasses.replace(cfg, patch=16), dataclasses.replace(cfg, heads=3),
           dataclasses.replace(cfg, hidden=1280, heads=10),          # head_dim 128 unsupported
           dataclasses.replace(cfg, std=(0.27, 0.0, 0.28)), dataclasses.replace(cfg, out_dim=100),
           dataclasses.replace(cfg, window_px=100), dataclasses.replace(cfg, layers=-1)]
    for b in bad:
        assert _status(lambda: B.VisionTower(b, lib)) == B.VIT_E_ARG, b
    assert lib.vit_create(None, ctypes.byref(B._P())) == B.VIT_E_ARG
    assert b"NULL" in lib.vit_last_error()
    for prec in ("f16", "bf16", "bf16x2", "bf16f8"):
        assert _status(lambda: B.VisionTower(cfg, lib, activation_precision=prec)) == B.VIT_OK, prec
    c = B.make_config(cfg)
    c.activation_precision = 4
    assert lib.vit_create(ctypes.byref(c), ctypes.byref(B._P())) == B.VIT_E_ARG
    assert b"activation_precision" in lib.vit_last_error()


def test_weight_validation_and_state(lib):
    t = B.VisionTower(tower_config(1), lib)
    t.load_weight("pe.w", np.zeros((64, 1176), np.float32))
    assert _status(lambda: t.load_weight("pe.w", np.zeros((64, 1176), np.float32))) == B.VIT_E_WEIGHTS
    assert _status(lambda: t.load_weight("x", np.zeros((0,), np.float32))) == B.VIT_E_SHAPE
    # encode before finalize is a state error, detected before any GPU work
    p = t.plan([[1, 4, 4]], [1])
    st = lib.vit_encode(t.handle, p.handle, 1, 256, 1 << 30, 256, None)
    assert st == B.VIT_E_STATE


@pytest.mark.parametrize("grid,frames,status", [
    ([[1, 3, 4]], [1], B.VIT_E_SHAPE),           # odd h
    ([[0, 4, 4]], [1], B.VIT_E_SHAPE),           # t = 0
    ([[2, 4, 4]], [1], B.VIT_E_SHAPE),           # image with t > 1
    ([[2, 4, 4]], [3], B.VIT_E_SHAPE),           # frames != 2t
    ([[1, 4, 4], [2, 6, 8]], [1, 4], B.VIT_OK),
])
def test_plan_validation(lib, grid, frames, status):
    t = B.VisionTower(tower_config(1), lib)
    assert _status(lambda: t.plan(grid, frames)) == status


def test_plan_rejects_batches_beyond_32bit_operand_addressing(lib):
    """Every GEMM / attention operand is addressed with 32-bit buffer offsets.  A batch whose
    largest operand would reach 2 GiB is refused by vit_plan_create (pure host), so it never
    fails half-way through an enqueued forward.  bf16 + e4m3 activations, GELU width 5120:
    the MLP activation [N][5120] bf16 crosses 2 GiB at N = 209,716 patches."""
    t = B.VisionTower(tower_config(3), lib, activation_precision="bf16f8")
    limit = (1 << 31) // (5120 * 2)            # largest N (multiple of 16) whose activation fits
    side = 2 * int(np.sqrt(limit / 4))         # an even square grid just below it
    ok = t.plan([[1, side, side]], [1])
    assert ok.n_patches == side * side < limit
    # the same patch count plus one more image of 16 rows of 2x2 units crosses the limit
    rows = (limit - side * side) // side + 2
    rows += rows % 2
    assert side * (side + rows) > limit
    assert _status(lambda: t.plan([[1, side, side], [1, rows, side]], [1, 1])) == B.VIT_E_SHAPE
    assert b"MLP activation" in lib.vit_last_error()
    # hi+lo pairs double the activation width: the limit halves
    t2 = B.VisionTower(tower_config(3), lib, activation_precision="bf16x2")
    assert _status(lambda: t2.plan([[1, side, side]], [1])) == B.VIT_E_SHAPE


def test_plan_rejects_video_frames_beyond_32bit_stride(lib):
    """A video frame of 2^31 bytes or more cannot be described by the unit descriptors'
    32-bit frame stride; the planner refuses it (the operand-extent check, which comes
    first, already covers every such frame at these tower widths)."""
    t = B.VisionTower(tower_config(4), lib)
    side = 2 * 1024                             # 28672 px square frames, 2.47 GB each
    assert 3 * (14 * side) ** 2 > (1 << 31)
    assert _status(lambda: t.plan([[1, side, side]], [2])) == B.VIT_E_SHAPE
    # an image of the same size is read once per slot and has no frame stride; it is still
    # refused, by the operand extents
    assert _status(lambda: t.plan([[1, side, side]], [1])) == B.VIT_E_SHAPE


def test_empty_batch_is_a_noop(lib):
    t = B.VisionTower(tower_config(1), lib)
    p = t.plan(np.zeros((0, 3), np.int32), np.zeros(0, np.int32))
    assert p.n_patches == 0 and p.out_rows == 0 and p.pixel_bytes == 0


def test_plan_sizes_and_identity_row_order(lib):
    t = B.VisionTower(tower_config(3), lib)
    grid = [[1, 82, 22], [1, 30, 34], [3, 6, 8]]
    p = t.plan(grid, [1, 1, 6])
    n = 82 * 22 + 30 * 34 + 3 * 6 * 8
    assert p.n_patches == n and p.out_rows == n // 4 and p.out_cols == 3584
    assert p.pixel_bytes == 3 * (82 * 14 * 22 * 14 + 30 * 14 * 34 * 14 + 6 * 6 * 14 * 8 * 14)
    assert np.array_equal(p.row_order(), np.arange(n))
    small = t.plan(grid[:1], [1])
    assert small.ws_bytes < p.ws_bytes


def test_window_order_matches_oracle_window_partition(lib):
    cfg = tower_config(5)
    t = B.VisionTower(cfg, lib)
    grid = np.array([[1, 24, 48], [1, 18, 28], [4, 18, 30]])
    frames = [1, 1, 8]
    p = t.plan(grid, frames)
    order = p.row_order()
    n = int((grid[:, 0] * grid[:, 1] * grid[:, 2]).sum())
    assert np.array_equal(np.sort(order), np.arange(n))          # a permutation
    # merge units stay whole and in (dh, dw) order
    assert np.all(order[0::4] % 4 == 0) and np.all(np.diff(order.reshape(-1, 4), axis=1) == 1)
    pos = O.patch_positions(grid)
    wins = O.window_segments(pos, cfg.window_px // cfg.patch)
    win_id = np.empty(n, np.int64)
    for i, s in enumerate(wins):
        win_id[s] = i
    ids = win_id[order]
    # each window is one contiguous run of internal rows
    runs = ids[np.r_[True, ids[1:] != ids[:-1]]]
    assert len(runs) == len(wins) and len(set(runs.tolist())) == len(wins)
    # items stay contiguous and in order
    assert np.all(np.diff(pos["item"][order]) >= 0)


def test_workspace_grows_with_batch(lib):
    t = B.VisionTower(tower_config(2), lib)
    sizes = [t.plan([[1, 2 * k, 2 * k]], [1]).ws_bytes for k in (2, 8, 16, 32)]
    assert sizes == sorted(sizes) and len(set(sizes)) == 4


# ---- attention work units and the planner's key splits (pure host)

def _check_units(plain, split, n_merge, n_parts):
    """The split list covers exactly the plain list's query blocks: each block either as its
    plain unit (partial slot -1) or as parts that tile its key blocks [0, nkb) in consecutive,
    distinct partial slots, each part at least 16 key blocks."""
    nkb = lambda L: (L + 31) // 32
    blocks = {}
    for u in plain:
        assert u[3] == 0 and u[4] == nkb(u[1]) and u[5] == -1
        blocks[(u[0], u[2])] = u
    seen, slots, merged = set(), set(), 0
    by_block = {}
    for u in split:
        key = (u[0], u[2])
        assert key in blocks and u[1] == blocks[key][1]
        by_block.setdefault(key, []).append(u)
    assert set(by_block) == set(blocks)
    for key, us in by_block.items():
        if len(us) == 1 and us[0][5] == -1:
            assert us[0][3] == 0 and us[0][4] == nkb(us[0][1])
            continue
        merged += 1
        us = sorted(us, key=lambda u: u[3])
        assert all(u[5] >= 0 for u in us)
        assert us[0][3] == 0 and us[-1][4] == nkb(us[0][1])
        assert all(a[4] == b[3] for a, b in zip(us, us[1:]))          # contiguous key ranges
        assert all(u[4] - u[3] >= 16 for u in us)
        sl = [u[5] for u in us]
        assert sl == list(range(sl[0], sl[0] + len(sl)))               # consecutive slots in key order
        assert not (set(sl) & slots) and all(0 <= x < n_parts for x in sl)
        slots |= set(sl)
    assert merged == n_merge and len(slots) == n_parts


def test_attention_units_and_key_splits(lib):
    # the 16-frame video (one 18,432-token segment): 72 query blocks per head, 2.25 rounds of
    # the 512 two-per-CU slots -- the planner splits the tail's key ranges
    t = B.VisionTower(tower_config(4), lib)
    p = t.plan([[8, 36, 64]], [16])
    plain, nm0, np0 = p.attention_units(split=False)
    split, nm, npart = p.attention_units(split=True)
    assert len(plain) == 72 and nm0 == 0 and np0 == 0
    assert nm > 0 and len(split) > len(plain)
    _check_units(plain, split, nm, npart)
    # a single 8-block query block cannot be split (parts of at least 16 blocks)
    small = t.plan([[1, 16, 16]], [1])
    u, nm, npart = small.attention_units()
    assert len(u) == 1 and nm == 0 and u[0][5] == -1
    # the 8-image batch shape: whatever the planner chose is a valid cover
    t3 = B.VisionTower(tower_config(3), lib)
    g = np.array([[1, 82, 22], [1, 30, 34], [1, 30, 80], [1, 86, 62], [1, 18, 22], [1, 42, 50], [1, 66, 54],
                  [1, 36, 28]], dtype=np.int32)
    p3 = t3.plan(g, np.ones(8, dtype=np.int32))
    _check_units(p3.attention_units(split=False)[0], *p3.attention_units(split=True))
    # window layers (1-wave units) are never split
    t5 = B.VisionTower(tower_config(5), lib)
    p5 = t5.plan([[1, 48, 64], [4, 32, 32]], [1, 8])
    w, nmw, _ = p5.attention_units(windows=True)
    assert nmw == 0
    with pytest.raises(B.VitError):
        p5.attention_units(windows=2)


def test_key_split_cover_on_random_batches(lib):
    # random mixes of images and videos (seeded): every split list is an exact cover
    rng = np.random.default_rng(11)
    t = B.VisionTower(tower_config(4), lib)
    splits = 0
    for _ in range(60):
        n = int(rng.integers(1, 9))
        grid, frames = [], []
        for _ in range(n):
            if rng.random() < 0.3:
                tt = int(rng.integers(1, 9))
                grid.append([tt, 2 * int(rng.integers(4, 40)), 2 * int(rng.integers(4, 40))])
                frames.append(2 * tt)
            else:
                grid.append([1, 2 * int(rng.integers(4, 60)), 2 * int(rng.integers(4, 60))])
                frames.append(1)
        p = t.plan(np.array(grid, dtype=np.int32), np.array(frames, dtype=np.int32))
        plain = p.attention_units(split=False)[0]
        split, nm, npart = p.attention_units(split=True)
        _check_units(plain, split, nm, npart)
        splits += nm > 0
    assert splits > 0   # the planner split some of them


# ---- premise of the two normalisation kernels (table vs one float32 fma per byte)

def _round_fraction(q, mant_bits):
    """Round a rational to the nearest binary float with `mant_bits` fraction bits (ties to even)."""
    from fractions import Fraction
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = 0
    while q >= 2:
        q /= 2
        e += 1
    while q < 1:
        q *= 2
        e -= 1
    m = q * 2 ** mant_bits
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * Fraction(fl) * Fraction(2) ** (e - mant_bits)


def _fma_path_mismatches(mean, std):
    """Bytes whose bf16(fp32 fma(x, fp32(1/(255 s)), fp32(-m/s))) differs from bf16 of the exact
    quotient ((x/255) - m)/s, with m and s the float32 values of the configured mean/std."""
    from fractions import Fraction
    bad = 0
    for c in range(3):
        m = Fraction(float(np.float32(mean[c])))
        s = Fraction(float(np.float32(std[c])))
        a = _round_fraction(1 / (255 * s), 23)
        b = _round_fraction(-m / s, 23)
        for x in range(256):
            exact = _round_fraction((Fraction(x, 255) - m) / s, 7)
            if _round_fraction(_round_fraction(x * a + b, 23), 7) != exact:
                bad += 1
    return bad


def test_normalisation_fma_path_premise():
    # the workloads' mean/std: the fma form rounds exactly like the table (fma kernel runs)
    cfg = tower_config(3)
    assert _fma_path_mismatches(cfg.mean, cfg.std) == 0
    # the table-path GPU test's mean/std: one byte differs, so the library keeps the table
    assert _fma_path_mismatches((0.1, 0.2, 0.3), (0.11, 0.13, 0.17)) >= 1


# ---- the header as a plain C interface: a C99 program compiled against include/vit.h and
# linked with the library runs the host-side calls (no GPU call is made)

_C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "vit.h"

int main(void) {
  vit_config c;
  memset(&c, 0, sizeof c);
  c.hidden = 64; c.heads = 2; c.layers = 1; c.mlp_dim = 256;
  c.mlp_kind = VIT_MLP_GELU; c.norm_kind = VIT_NORM_LAYER; c.norm_eps = 1e-6f;
  c.patch = 14; c.temporal_patch = 2; c.merge = 2; c.out_dim = 128; c.rope_theta = 10000.f;
  for (int i = 0; i < 3; ++i) { c.mean[i] = 0.5f; c.std[i] = 0.25f; }
  c.activation_precision = VIT_ACT_F16;
  vit_ctx* ctx = NULL;
  if (vit_create(&c, &ctx) != VIT_OK) { printf("create: %s\n", vit_last_error()); return 1; }
  const int32_t grid[6] = {1, 4, 6, 2, 2, 2};   /* a 56 x 84 image and a 4-frame 28 x 28 clip */
  const int32_t frames[2] = {1, 4};
  vit_plan* plan = NULL;
  if (vit_plan_create(ctx, grid, frames, 2, &plan) != VIT_OK) { printf("plan: %s\n", vit_last_error()); return 1; }
  size_t px = 0, ws = 0;
  int64_t rows = 0, cols = 0, n = 0;
  if (vit_plan_sizes(plan, &px, &ws, &rows, &cols) != VIT_OK || vit_plan_rows(plan, &n, NULL) != VIT_OK) return 1;
  printf("pixels %zu rows %lld cols %lld patches %lld ws %d\n", px, (long long)rows, (long long)cols,
         (long long)n, ws > 0);
  vit_config bad = c;
  bad.heads = 3;   /* 64 / 3 is no head size */
  vit_ctx* ctx2 = NULL;
  const vit_status s = vit_create(&bad, &ctx2);
  printf("bad config %d %d %d\n", (int)s, ctx2 == NULL, (int)(strlen(vit_last_error()) > 0));
  vit_plan_destroy(plan);
  vit_destroy(ctx);
  return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_vit.c"
    src.write_text(_C_PROGRAM)
    exe = tmp_path / "use_vit"
    lib = os.path.abspath(B.LIB_PATH)
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(B.__file__))), "include")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", inc, str(src), "-o", str(exe), lib,
                    f"-Wl,-rpath,{os.path.dirname(lib)}"], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.split("\n")
    # 56 x 84 px image: 4 x 6 patches; 4-frame 28 x 28 clip: 2 temporal x 2 x 2 patches
    assert out[0] == f"pixels {56 * 84 * 3 + 4 * 28 * 28 * 3} rows {(24 + 8) // 4} cols 128 patches 32 ws 1"
    assert out[1] == f"bad config {B.VIT_E_ARG} 1 1"
