"""Pins for the CPU oracle: each test ties one oracle step to something other
than the oracle itself -- exact rational arithmetic, a torch library routine
(conv3d/conv2d, layer_norm, rms_norm, scaled_dot_product_attention,
TransformerEncoderLayer), a closed form, an invariant, brute force on a tiny
input, or a value the pages print.  All CPU, no GPU."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import vit_oracle as O
from workloads import TowerConfig, make_custom_workload, tower_config

MEAN = (0.48, 0.46, 0.41)
STD = (0.27, 0.26, 0.28)


# ---------------------------------------------------------------- normalise


def _bf16_exact(v: Fraction) -> Fraction:
    """bfloat16 round-to-nearest-even of an exact rational (8 significant bits)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    scaled = a / ulp                      # in [128, 256)
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def test_normalize_table_is_exact_rounding_of_exact_quotient():
    table = O.normalize_table(MEAN, STD)
    worst = 1.0
    for c in range(3):
        m = Fraction(float(np.float32(MEAN[c])))
        s = Fraction(float(np.float32(STD[c])))
        for x in range(256):
            exact = (Fraction(x, 255) - m) / s
            want = _bf16_exact(exact)
            assert Fraction(float(table[c][x])) == want, (c, x)
            # distance of the exact value from the nearest rounding midpoint, relative
            a = abs(exact)
            e = math.floor(math.log2(float(a))) if a else 0
            ulp = Fraction(2) ** (e - 7)
            frac = (a / ulp) - math.floor(a / ulp)
            worst = min(worst, abs(float(frac) - 0.5) * float(ulp / a) if a else 1.0)
    assert worst > 2.0 ** -40          # no value sits on a float64-ambiguous midpoint


def test_bf16_round_matches_torch_on_float32_inputs():
    g = np.random.default_rng(0)
    v = (g.standard_normal(100000) * np.exp(g.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(v.astype(np.float64)), ref)


def test_uint8_values_are_exact_in_bf16():
    x = np.arange(256, dtype=np.float64)
    assert np.array_equal(O.bf16_round(x), x)


def test_normalize_closed_form_spot_values():
    table = O.normalize_table(MEAN, STD)
    for c in range(3):
        m, s = float(np.float32(MEAN[c])), float(np.float32(STD[c]))
        assert table[c][0] == float(_bf16_exact(Fraction(-m) / Fraction(s)))
        assert table[c][255] == float(_bf16_exact((1 - Fraction(m)) / Fraction(s)))


def test_rescale_by_factor_equals_divide_by_255():
    # the pages show rescale both as a division and as a multiply by a factor
    table = O.normalize_table(MEAN, STD)
    x = np.arange(256, dtype=np.float64)
    for c in range(3):
        m, s = float(np.float32(MEAN[c])), float(np.float32(STD[c]))
        alt = O.bf16_round((x * (1.0 / 255.0) - m) / s)
        assert np.array_equal(alt, table[c])


def test_double_normalisation_is_visible():
    table = O.normalize_table(MEAN, STD)
    once = table[0]
    twice = O.bf16_round((once / 255.0 - float(np.float32(MEAN[0]))) / float(np.float32(STD[0])))
    assert np.abs(once - twice).max() > 1.0


# ---------------------------------------------------------------- patchify + embed


def _clip_items():
    g = np.random.default_rng(7)
    img = g.integers(0, 256, size=(1, 56, 84, 3), dtype=np.uint8)
    vid = g.integers(0, 256, size=(4, 28, 56, 3), dtype=np.uint8)
    return [img, vid], np.array([[1, 4, 6], [2, 2, 4]])


def test_patch_embed_equals_conv3d_and_merge_order():
    frames, grid = _clip_items()
    table = O.normalize_table(MEAN, STD)
    x = O.patchify(frames, grid, table)
    assert x.shape == (24 + 16, 1176)
    g = np.random.default_rng(8)
    d = 6
    w = g.standard_normal((d, 3, 2, 14, 14))
    rows = O.patch_embed(x, w)
    seen = []
    base = 0
    for n, fr in enumerate(frames):
        clip = O.item_clip(fr)                                       # [F][H][W][3]
        normed = np.stack([table[c][clip[..., c]] for c in range(3)], axis=-1)
        vol = torch.from_numpy(normed.transpose(3, 0, 1, 2)[None].copy())   # [1][C][F][H][W]
        y = F.conv3d(vol, torch.from_numpy(w), stride=(2, 14, 14))[0].numpy()  # [d][T][h][w]
        t, h, ww = grid[n]
        cols = y.reshape(d, -1).T                                   # (t, ph, pw) row-major
        for k in range(t * h * ww):
            r = rows[base + k]
            hit = np.flatnonzero(np.abs(cols - r).max(axis=1) < 1e-9)
            assert hit.size == 1
            ti, rem = divmod(int(hit[0]), h * ww)
            seen.append((n, ti, *divmod(rem, ww)))
        base += t * h * ww
    # merge units: 4 consecutive rows are one 2x2 block, row-major inside; blocks row-major; t outermost
    for k in range(0, len(seen), 4):
        n, t, ph, pw = seen[k]
        assert ph % 2 == 0 and pw % 2 == 0
        assert seen[k:k + 4] == [(n, t, ph, pw), (n, t, ph, pw + 1), (n, t, ph + 1, pw), (n, t, ph + 1, pw + 1)]
    blocks = [s for s in seen[::4]]
    assert blocks == sorted(blocks)
    pos = O.patch_positions(grid)
    assert list(zip(pos["item"], pos["t"], pos["hpos"], pos["wpos"])) == seen


def test_image_frame_duplication_equals_summed_temporal_kernel():
    frames, grid = _clip_items()
    table = O.normalize_table(MEAN, STD)
    x = O.patchify(frames[:1], grid[:1], table)
    g = np.random.default_rng(9)
    w = g.standard_normal((4, 3, 2, 14, 14))
    rows = O.patch_embed(x, w)
    normed = np.stack([table[c][frames[0][0][..., c]] for c in range(3)], axis=0)[None]
    y = F.conv2d(torch.from_numpy(normed.copy()), torch.from_numpy(w.sum(axis=2)), stride=14)[0].numpy()
    pos = O.patch_positions(grid[:1])
    want = y[:, pos["hpos"], pos["wpos"]].T
    assert np.allclose(rows, want, rtol=0, atol=1e-10)


def test_shapes_printed_on_the_pages(golden_dir):
    with open(os.path.join(golden_dir, "shapes.json")) as f:
        ex = json.load(f)["example"]
    grid = np.array(ex["grid_thw"])
    g = np.random.default_rng(1)
    frames = [g.integers(0, 256, size=(2 * t if t > 1 else 1, 14 * h, 14 * w, 3), dtype=np.uint8)
              for t, h, w in grid]
    x = O.patchify(frames, grid, O.normalize_table(MEAN, STD))
    assert x.shape == (ex["num_patches"], ex["features"])
    pos = O.patch_positions(grid)
    assert pos["hpos"].shape == (ex["num_patches"],)
    ang = O.rope_angles(pos["hpos"], pos["wpos"], ex["head_dim"])
    assert ang.shape == (ex["num_patches"], ex["rotary_dim"])


# ---------------------------------------------------------------- RoPE


def _rope_inputs(n=12, heads=3, hd=80, seed=3):
    g = np.random.default_rng(seed)
    return g.standard_normal((n, heads, hd)), g.integers(0, 40, n), g.integers(0, 40, n)


def test_rope_preserves_norm_and_zero_is_identity():
    x, hp, wp = _rope_inputs()
    y = O.apply_rope(x, O.rope_angles(hp, wp, 80))
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    z = O.apply_rope(x, O.rope_angles(0 * hp, 0 * wp, 80))
    assert np.array_equal(z, x)


def test_rope_relative_position():
    x, hp, wp = _rope_inputs()
    q, k = x[:6], x[6:]
    def dots(dh, dw):
        a = O.apply_rope(q, O.rope_angles(hp[:6] + dh, wp[:6] + dw, 80))
        b = O.apply_rope(k, O.rope_angles(hp[6:] + dh, wp[6:] + dw, 80))
        return np.einsum("ihd,jhd->ijh", a, b)
    assert np.allclose(dots(0, 0), dots(5, 11), rtol=1e-10, atol=1e-10)
    assert not np.allclose(dots(0, 0), dots(0, 0) * 0 + np.einsum("ihd,jhd->ijh", q, k))


def test_rope_first_half_from_rows_second_half_from_columns(golden_dir):
    with open(os.path.join(golden_dir, "rope_lookup_example.json")) as f:
        ex = json.load(f)
    hp, wp = ex["position"]
    a = O.rope_angles(np.array([hp]), np.array([wp]), 80)[0]
    cache_h = O.rope_angles(np.array([ex["row_axis_cache_index"]]), np.array([0]), 80)[0]
    cache_w = O.rope_angles(np.array([0]), np.array([ex["col_axis_cache_index"]]), 80)[0]
    half = 20
    assert np.array_equal(a[:half], cache_h[:half]) and np.all(cache_h[half:] == 0)
    assert np.array_equal(a[half:], cache_w[half:]) and np.all(cache_w[:half] == 0)
    # moving only the column position leaves the row-axis slots untouched
    x, _, _ = _rope_inputs(n=1)
    y1 = O.apply_rope(x, O.rope_angles(np.array([hp]), np.array([wp]), 80))
    y2 = O.apply_rope(x, O.rope_angles(np.array([hp]), np.array([wp + 7]), 80))
    for k in range(half):
        assert np.array_equal(y1[..., k], y2[..., k]) and np.array_equal(y1[..., k + 40], y2[..., k + 40])


def test_rope_is_complex_rotation_of_half_pairs():
    x, hp, wp = _rope_inputs()
    ang = O.rope_angles(hp, wp, 80)
    z = (x[..., :40] + 1j * x[..., 40:]) * np.exp(1j * ang)[:, None, :]
    y = O.apply_rope(x, ang)
    assert np.allclose(y[..., :40], z.real, atol=1e-13) and np.allclose(y[..., 40:], z.imag, atol=1e-13)


def test_rope_frequencies_closed_form():
    ang = O.rope_angles(np.array([1]), np.array([1]), 80)[0]
    assert ang[0] == 1.0 and ang[20] == 1.0
    assert math.isclose(ang[19], 10000.0 ** (-38 / 40), rel_tol=1e-15)


# ---------------------------------------------------------------- norms, activations


def test_norms_and_activations_match_torch():
    g = np.random.default_rng(4)
    x = g.standard_normal((7, 64)) * 3 + 1
    w = 1 + 0.1 * g.standard_normal(64)
    b = 0.1 * g.standard_normal(64)
    tx = torch.from_numpy(x)
    assert np.allclose(O.layer_norm(x, w, b, 1e-6),
                       F.layer_norm(tx, (64,), torch.from_numpy(w), torch.from_numpy(b), 1e-6).numpy(),
                       atol=1e-12)
    assert np.allclose(O.rms_norm(x, w, 1e-6),
                       F.rms_norm(tx, (64,), torch.from_numpy(w), 1e-6).numpy(), atol=1e-12)
    assert np.allclose(O.gelu(x), F.gelu(tx).numpy(), atol=1e-13)
    assert np.allclose(O.silu(x), F.silu(tx).numpy(), atol=1e-13)
    y = O.layer_norm(x, np.ones(64), np.zeros(64), 0.0)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-13) and np.allclose(y.var(axis=1), 1, atol=1e-12)
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, atol=1e-13)


# ---------------------------------------------------------------- attention


def _attn_inputs(lengths, heads=2, hd=8, seed=5):
    g = np.random.default_rng(seed)
    n = sum(lengths)
    q, k, v = (g.standard_normal((n, heads, hd)) for _ in range(3))
    cu = np.cumsum([0] + list(lengths))
    segs = [np.arange(cu[i], cu[i + 1]) for i in range(len(lengths))]
    return q, k, v, segs, cu


def test_attention_matches_torch_sdpa_with_block_diagonal_mask():
    q, k, v, segs, cu = _attn_inputs([5, 1, 9, 3])
    n = q.shape[0]
    mask = np.zeros((n, n), dtype=bool)
    for s in segs:
        mask[np.ix_(s, s)] = True
    ref = F.scaled_dot_product_attention(torch.from_numpy(q.transpose(1, 0, 2)), torch.from_numpy(k.transpose(1, 0, 2)),
                                         torch.from_numpy(v.transpose(1, 0, 2)),
                                         attn_mask=torch.from_numpy(mask)).numpy().transpose(1, 0, 2)
    assert np.allclose(O.attention(q, k, v, segs), ref, atol=1e-13)


def test_attention_brute_force_loops():
    q, k, v, segs, _ = _attn_inputs([3, 4], heads=1, hd=4)
    out = O.attention(q, k, v, segs)
    for s in segs:
        for i in s:
            e = [math.exp(sum(q[i, 0, d] * k[j, 0, d] for d in range(4)) / 2.0) for j in s]
            tot = sum(e)
            for d in range(4):
                assert math.isclose(out[i, 0, d], sum(e[a] * v[j, 0, d] for a, j in enumerate(s)) / tot,
                                    rel_tol=1e-12, abs_tol=1e-13)


def test_attention_isolation_degenerate_cases_and_row_subset():
    q, k, v, segs, cu = _attn_inputs([6, 1, 7])
    out = O.attention(q, k, v, segs)
    assert np.array_equal(out[6], v[6])                               # one-token segment: O = V
    q2 = q.copy(); k2 = k.copy(); v2 = v.copy()
    q2[7:], k2[7:], v2[7:] = 0.0, 5.0, -1.0                           # perturb item 2
    out2 = O.attention(q2, k2, v2, segs)
    assert np.array_equal(out2[:7], out[:7])
    assert np.allclose(out2[7:], -1.0)
    qz = np.zeros_like(q)
    oz = O.attention(qz, k, v, segs)
    assert np.allclose(oz[:6], v[:6].mean(axis=0, keepdims=True), atol=1e-14)
    rows = np.array([12, 0, 7])
    assert np.allclose(O.attention(q, k, v, segs, rows=rows), out[rows], atol=1e-14)


def test_window_segments_partition_and_large_window_is_per_frame():
    pos = O.patch_positions(np.array([[2, 10, 6], [1, 4, 4]]))
    segs = O.window_segments(pos, 4)
    allrows = np.sort(np.concatenate(segs))
    assert np.array_equal(allrows, np.arange(len(pos["item"])))
    for s in segs:
        assert len(s) <= 16
        for key in ("item", "t"):
            assert np.unique(pos[key][s]).size == 1
        assert np.unique(pos["hpos"][s] // 4).size == 1 and np.unique(pos["wpos"][s] // 4).size == 1
    assert sorted(len(s) for s in segs if pos["item"][s[0]] == 0) == sorted([16, 8] * 2 * 2 + [8, 4] * 2)
    big = O.window_segments(pos, 100)
    assert len(big) == 3 and sorted(len(s) for s in big) == [16, 60, 60]


def test_window_mask_equals_permuted_contiguous_windows():
    pos = O.patch_positions(np.array([[1, 12, 8]]))
    segs = O.window_segments(pos, 4)
    g = np.random.default_rng(6)
    n = len(pos["item"])
    q, k, v = (g.standard_normal((n, 2, 8)) for _ in range(3))
    perm = np.concatenate(segs)
    cu = np.cumsum([0] + [len(s) for s in segs])
    contiguous = [np.arange(cu[i], cu[i + 1]) for i in range(len(segs))]
    o_perm = O.attention(q[perm], k[perm], v[perm], contiguous)
    o = O.attention(q, k, v, segs)
    assert np.allclose(o[perm], o_perm, atol=1e-14)


def _segments_by_key(keys):
    """Brute force: rows grouped by equal key tuples, as sorted row-index sets."""
    groups = {}
    for row, key in enumerate(keys):
        groups.setdefault(tuple(int(v) for v in key), []).append(row)
    return sorted(tuple(g) for g in groups.values())


def _as_sets(segs):
    return sorted(tuple(sorted(int(r) for r in s)) for s in segs)


def test_layer_schedule_full_layers_7_15_23_31_else_windows():
    """The Qwen2.5-shaped workload: 112 px windows in every layer except the full-attention
    layers 7, 15, 23 and 31 (0-based, as the workload states them).  Expected segments are
    built here by brute force from each row's (item, frame, window) or item alone; an
    inverted, shifted (1-based) or missing schedule fails."""
    cfg = tower_config(5)
    assert cfg.layers == 32 and tuple(cfg.full_attn_layers) == (7, 15, 23, 31)
    grid = np.array([[1, 18, 22], [2, 10, 6], [1, 4, 4]])
    pos = O.patch_positions(grid)
    wp = cfg.window_px // cfg.patch
    n = len(pos["item"])
    by_item = _segments_by_key([(pos["item"][r],) for r in range(n)])
    by_window = _segments_by_key([(pos["item"][r], pos["t"][r], pos["hpos"][r] // wp, pos["wpos"][r] // wp)
                                  for r in range(n)])
    assert len(by_item) == 3 and len(by_window) == 3 * 3 + 2 * (2 * 1) + 1   # ceil(h/8) * ceil(w/8) per frame
    full = []
    for layer in range(cfg.layers):
        got = _as_sets(O.layer_segments(layer, cfg, pos))
        if got == by_item:
            full.append(layer)
        else:
            assert got == by_window, f"layer {layer}: neither item nor window segments"
    assert full == [7, 15, 23, 31]
    # a tower without windows attends over whole items in every layer
    cfg3 = tower_config(3)
    assert all(_as_sets(O.layer_segments(l, cfg3, pos)) == by_item for l in (0, 7, 31))


def test_forward_applies_the_layer_schedule():
    """forward() on a 2-layer window tower (layer 1 full) equals two blocks composed by hand
    with brute-force segments: windows in layer 0, whole items in layer 1."""
    cfg = _tiny_cfg(layers=2, window_px=56, full_attn_layers=(1,), mlp_kind="swiglu", norm_kind="rms")
    wl = make_custom_workload(cfg, [(1, 112, 84), (2, 84, 56)], seed=23)
    x = O.patchify([it.frames for it in wl.items], wl.grid_thw, O.normalize_table(cfg.mean, cfg.std))
    pos = O.patch_positions(wl.grid_thw)
    ang = O.rope_angles(pos["hpos"], pos["wpos"], cfg.head_dim)
    n = len(pos["item"])
    wp = cfg.window_px // cfg.patch
    win = [np.array(s) for s in _segments_by_key(
        [(pos["item"][r], pos["t"][r], pos["hpos"][r] // wp, pos["wpos"][r] // wp) for r in range(n)])]
    items = [np.array(s) for s in _segments_by_key([(pos["item"][r],) for r in range(n)])]
    assert len(win) > len(items)
    r = O.patch_embed(x, wl.weights["pe.w"].astype(np.float64))
    r = O.block(r, wl.weights, 0, cfg, ang, win)
    r = O.block(r, wl.weights, 1, cfg, ang, items)
    want = O.merger(r, wl.weights, cfg)
    assert np.allclose(O.forward_workload(wl), want, rtol=0, atol=1e-12)
    # and the schedule matters: swapping the two layers' segments changes the output
    r2 = O.patch_embed(x, wl.weights["pe.w"].astype(np.float64))
    r2 = O.block(r2, wl.weights, 0, cfg, ang, items)
    r2 = O.block(r2, wl.weights, 1, cfg, ang, win)
    assert not np.allclose(O.merger(r2, wl.weights, cfg), want, atol=1e-6)


# ---------------------------------------------------------------- block, merger, tower


def _tiny_cfg(**kw):
    base = dict(hidden=32, heads=2, layers=2, mlp_dim=48, mlp_kind="gelu", norm_kind="layer", out_dim=24,
                weight_dtype="f32")
    base.update(kw)
    return TowerConfig("tiny-test", **base)


def test_block_matches_torch_transformer_encoder_layer_without_rope():
    cfg = _tiny_cfg()
    wl = make_custom_workload(cfg, [(1, 28 * 2, 28 * 3), (1, 28, 28)], seed=11)
    W = {k: v.astype(np.float64) for k, v in wl.weights.items()}
    g = np.random.default_rng(12)
    lens = [24, 4]
    r = g.standard_normal((sum(lens), cfg.hidden))
    segs = [np.arange(0, 24), np.arange(24, 28)]
    zero_angles = np.zeros((28, cfg.head_dim // 2))
    out = O.block(r, W, 0, cfg, zero_angles, segs)
    layer = torch.nn.TransformerEncoderLayer(cfg.hidden, cfg.heads, cfg.mlp_dim, dropout=0.0,
                                             activation="gelu", layer_norm_eps=cfg.norm_eps,
                                             batch_first=True, norm_first=True).double().eval()
    sd = {"self_attn.in_proj_weight": W["blk0.qkv.w"], "self_attn.in_proj_bias": W["blk0.qkv.b"],
          "self_attn.out_proj.weight": W["blk0.proj.w"], "self_attn.out_proj.bias": W["blk0.proj.b"],
          "linear1.weight": W["blk0.fc1.w"], "linear1.bias": W["blk0.fc1.b"],
          "linear2.weight": W["blk0.fc2.w"], "linear2.bias": W["blk0.fc2.b"],
          "norm1.weight": W["blk0.n1.g"], "norm1.bias": W["blk0.n1.b"],
          "norm2.weight": W["blk0.n2.g"], "norm2.bias": W["blk0.n2.b"]}
    layer.load_state_dict({k: torch.from_numpy(v.copy()) for k, v in sd.items()})
    with torch.no_grad():
        for s in segs:
            ref = layer(torch.from_numpy(r[s][None].copy()))[0].numpy()
            assert np.allclose(out[s], ref, atol=1e-12)
    # with real positions the block differs (RoPE is applied)
    pos = O.patch_positions(wl.grid_thw)
    ang = O.rope_angles(pos["hpos"], pos["wpos"], cfg.head_dim)
    assert not np.allclose(O.block(r, W, 0, cfg, ang, segs), out)


def test_swiglu_rms_block_matches_torch_functional():
    cfg = _tiny_cfg(mlp_kind="swiglu", norm_kind="rms", mlp_dim=40)
    wl = make_custom_workload(cfg, [(1, 56, 56)], seed=13)
    W = {k: torch.from_numpy(v.astype(np.float64)) for k, v in wl.weights.items()}
    g = np.random.default_rng(14)
    r = g.standard_normal((16, cfg.hidden))
    pos = O.patch_positions(wl.grid_thw)
    ang = O.rope_angles(pos["hpos"], pos["wpos"], cfg.head_dim)
    out = O.block(r, {k: v.numpy() for k, v in W.items()}, 0, cfg, ang, [np.arange(16)])
    tr = torch.from_numpy(r)
    h = F.rms_norm(tr, (32,), W["blk0.n1.g"], 1e-6)
    qkv = F.linear(h, W["blk0.qkv.w"], W["blk0.qkv.b"]).view(16, 3, 2, 16)
    c, s = torch.cos(torch.from_numpy(ang)), torch.sin(torch.from_numpy(ang))
    def rot(x):   # complex form of the pair rotation
        z = torch.complex(x[..., :8], x[..., 8:]) * torch.complex(c, s)[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)
    q, k, v = rot(qkv[:, 0]), rot(qkv[:, 1]), qkv[:, 2]
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1))
    r1 = tr + F.linear(o.transpose(0, 1).reshape(16, 32), W["blk0.proj.w"], W["blk0.proj.b"])
    h2 = F.rms_norm(r1, (32,), W["blk0.n2.g"], 1e-6)
    m = F.linear(F.silu(F.linear(h2, W["blk0.gate.w"], W["blk0.gate.b"])) * F.linear(h2, W["blk0.up.w"], W["blk0.up.b"]),
                 W["blk0.down.w"], W["blk0.down.b"])
    assert np.allclose(out, (r1 + m).numpy(), atol=1e-12)


def test_merger_concatenates_four_rows_and_matches_torch_mlp():
    cfg = _tiny_cfg()
    wl = make_custom_workload(cfg, [(1, 56, 56)], seed=15)
    W = {k: v.astype(np.float64) for k, v in wl.weights.items()}
    g = np.random.default_rng(16)
    r = g.standard_normal((16, 32))
    trace = {}
    z = O.merger(r, W, cfg, trace=trace)
    u = O.layer_norm(r, W["mrg.nq.g"], W["mrg.nq.b"], 1e-6)
    for k in range(4):
        for j in range(128):
            assert trace["u"][k, j] == u[4 * k + j // 32, j % 32]
    tu = F.layer_norm(torch.from_numpy(r), (32,), torch.from_numpy(W["mrg.nq.g"]), torch.from_numpy(W["mrg.nq.b"]), 1e-6)
    mlp = torch.nn.Sequential(torch.nn.Linear(128, 128), torch.nn.GELU(), torch.nn.Linear(128, 24)).double()
    mlp.load_state_dict({"0.weight": torch.from_numpy(W["mrg.fc1.w"]), "0.bias": torch.from_numpy(W["mrg.fc1.b"]),
                         "2.weight": torch.from_numpy(W["mrg.fc2.w"]), "2.bias": torch.from_numpy(W["mrg.fc2.b"])})
    with torch.no_grad():
        assert np.allclose(z, mlp(tu.reshape(4, 128)).numpy(), atol=1e-12)


def test_zero_block_weights_make_every_block_the_identity():
    cfg = _tiny_cfg(layers=3)
    wl = make_custom_workload(cfg, [(1, 56, 28), (4, 28, 28)], seed=17)
    W = dict(wl.weights)
    for name in list(W):
        if name.startswith("blk") and (name.endswith(".w") or name.endswith(".b")) and ".n" not in name:
            W[name] = np.zeros_like(W[name])
    frames = [it.frames for it in wl.items]
    out3 = O.forward(frames, wl.grid_thw, cfg, W)
    out0 = O.forward(frames, wl.grid_thw, cfg, W, layers=0)
    assert np.array_equal(out3, out0)
    x = O.patchify(frames, wl.grid_thw, O.normalize_table(cfg.mean, cfg.std))
    assert np.allclose(out0, O.merger(O.patch_embed(x, W["pe.w"].astype(np.float64)), W, cfg), atol=0)


def test_items_are_independent_through_the_tower():
    cfg = _tiny_cfg(layers=2)
    wl = make_custom_workload(cfg, [(1, 56, 28), (1, 28, 56), (2, 28, 28)], seed=19)
    full = O.forward_workload(wl)
    sub = O.forward_workload(wl, items=[1])
    assert np.allclose(full[2:4], sub, atol=1e-13)
    assert full.shape == (2 + 2 + 1, cfg.out_dim)


def test_tiny_workload_forward_shape():
    from workloads import make_workload
    wl = make_workload(1)
    out = O.forward_workload(wl)
    assert out.shape == (4, 128) and np.all(np.isfinite(out))
    cfg5 = tower_config(5)
    assert cfg5.window_px // cfg5.patch == 8


# ------------------------------------------------------------------ pixel content key (embedding cache)

def test_pixel_key_mix_is_splitmix64():
    """The finaliser reproduces the published SplitMix64 outputs from seed 0."""
    from oracle import pixel_key as PK
    got = [int(v) for v in PK.splitmix64_stream(0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_pixel_key_sensitivity_and_position():
    """One changed byte, two swapped words or a different length change both lanes; equal
    content gives equal keys."""
    from oracle import pixel_key as PK
    g = np.random.default_rng(11)
    x = g.integers(0, 256, size=(1, 56, 28, 3), dtype=np.uint8)
    k = PK.item_key(x)
    assert PK.item_key(x.copy()) == k
    y = x.copy()
    y[0, 10, 3, 1] ^= 1
    ky = PK.item_key(y)
    assert ky[0] != k[0] and ky[1] != k[1]
    w = x.reshape(-1).view("<u8").copy()
    w[[0, 1]] = w[[1, 0]]
    kw = PK.item_key(w.view(np.uint8))
    if w[0] != w[1]:
        assert kw[0] != k[0] and kw[1] != k[1]
    z = np.concatenate([x.reshape(-1), np.zeros(16, np.uint8)])
    kz = PK.item_key(z)
    assert kz[0] != k[0] and kz[1] != k[1]


# ------------------------------------------------------------------ device resize (before the path)

def test_resize_side_rule():
    from oracle import resize as RS
    assert [RS.resize_side(s) for s in (1, 13, 41, 42, 55, 56, 69, 70, 1344, 1000)] == \
        [28, 28, 28, 56, 56, 56, 56, 84, 1344, 1008]


def test_resize_identity_constant_and_closed_form():
    from oracle import resize as RS
    g = np.random.default_rng(5)
    x = g.integers(0, 256, size=(2, 56, 84, 3), dtype=np.uint8)
    assert np.array_equal(RS.resize(x), x)                      # already on the grid
    c = np.full((1, 37, 61, 3), 173, np.uint8)
    assert np.all(RS.resize(c) == 173)                          # constant stays constant
    # 14 -> 28 (2x): output d samples s = d/2 - 1/4; on the ramp p_k = 16 k that is 16 s =
    # 8 d - 4 inside, with d = 0 clamped to p_0 and d = 27 to p_13
    ramp = np.zeros((1, 14, 14, 3), np.uint8)
    ramp[0] = (16 * np.arange(14, dtype=np.uint8))[None, :, None]
    out = RS.resize(ramp)[0, 5, :, 0]
    assert out.tolist() == [0] + [8 * d - 4 for d in range(1, 27)] + [208]
    # a single bright column spreads over its two nearest output columns on each side
    spot = np.zeros((1, 14, 14, 3), np.uint8)
    spot[0, :, 1] = 200
    assert RS.resize(spot)[0, 0, :6, 0].tolist() == [0, 50, 150, 150, 50, 0]



def test_resize_matches_per_pixel_exact_rationals():
    """The vectorised integer oracle against a per-pixel evaluation of the rule in exact
    rationals on small off-grid images (down: 41 -> 28, 47 -> 56 up, 69 -> 56)."""
    from oracle import resize as RS
    g = np.random.default_rng(6)

    def ref(frames):
        F, H, W, _ = frames.shape
        dh, dw = RS.resize_side(H), RS.resize_side(W)

        def ax(d, D, S):
            s = Fraction(2 * d + 1, 2) * Fraction(S, D) - Fraction(1, 2)
            if s <= 0:
                return 0, 0, 0
            i0 = math.floor(s)
            if i0 >= S - 1:
                return S - 1, S - 1, 0
            return i0, i0 + 1, math.floor((s - i0) * 2048 + Fraction(1, 2))

        out = np.zeros((F, dh, dw, 3), np.uint8)
        for f in range(F):
            for y in range(dh):
                y0, y1, wy = ax(y, dh, H)
                for x in range(dw):
                    x0, x1, wx = ax(x, dw, W)
                    for c in range(3):
                        top = (2048 - wx) * int(frames[f, y0, x0, c]) + wx * int(frames[f, y0, x1, c])
                        bot = (2048 - wx) * int(frames[f, y1, x0, c]) + wx * int(frames[f, y1, x1, c])
                        out[f, y, x, c] = ((2048 - wy) * top + wy * bot + (1 << 21)) >> 22
        return out

    for h, w in ((41, 47), (69, 30), (29, 83)):
        x = g.integers(0, 256, size=(1, h, w, 3), dtype=np.uint8)
        assert np.array_equal(RS.resize(x), ref(x)), (h, w)
