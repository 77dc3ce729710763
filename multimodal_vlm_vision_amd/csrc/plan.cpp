// Host planner: validates a batch and builds every piece of per-forward
// metadata once (no GPU call).  What it encodes:
//  - merge-unit order of patch rows, with each 2x2 unit's four rows adjacent
//    and the T temporal patches of an item concatenated ("vLLM multimodal
//    inference | ViT performance optimisation", sections 2.2 and 3.3);
//  - per-row (hpos, wpos) for the 2D rotary embedding and the cos/sin cache
//    of max(h, w) positions (same blog, section 3.3);
//  - window-attention order for towers with windows (section 3.3 names the
//    reorder; the window geometry is a reading: square windows of
//    window_px / 14 patches per frame, tiled from the top-left, truncated at
//    the edges, units row-major inside a window);
//  - segment bounds for block-diagonal attention, computed once per forward
//    and shared by every layer (section 3.4), as attention work lists.
#include <algorithm>
#include <climits>
#include <functional>
#include <cmath>
#include <cstring>

#include "vit_internal.h"

namespace vitmi {

namespace {

template <class T>
int64_t put(std::vector<uint8_t>& blob, const std::vector<T>& v) {
  int64_t off = round_up((int64_t)blob.size(), 256);
  blob.resize(off + v.size() * sizeof(T));
  if (!v.empty()) std::memcpy(blob.data() + off, v.data(), v.size() * sizeof(T));
  return off;
}

struct Seg {
  int32_t start, len;
};

// ---- key splits of the long units.  The 4-wave attention workgroups run two per CU and are
// dispatched in work order, each XCD (workgroups go round-robin over 8 XCDs) taking a
// contiguous range of (head, unit) pairs, head-major.  A list-scheduling model of that
// dispatch (a unit costs its key blocks plus a fixed overhead) finds the unit that finishes
// last; while the modelled makespan exceeds the mean load per slot by more than 3%, that unit
// is split into two halves of its key range (no part below kMinPartBlocks blocks), and the
// list is kept largest-first.  The best list found is kept only if its makespan plus the
// merge pass's modelled cost is at least 3% below the unsplit makespan.  (Units of time: one
// key block of one 4-wave workgroup, ~1.4 us on MI355X with two workgroups per CU; the merge
// moves (head_dim + 2) x 1 KB per partial slot and head, at a few TB/s, plus a launch.)
constexpr int kAttnQB = 256;            // queries per long unit
constexpr int kAttnKB = 32;             // keys per block
constexpr int kMinPartBlocks = 16;
constexpr double kUnitOverhead = 4.0;   // key blocks' worth of per-unit work (query load, output)
constexpr double kPartOverhead = 2.0;   // extra for a part (its partial store)
constexpr double kMergeFixed = 3.0;     // merge launch
constexpr double kMergePerSlot = 0.015; // merge traffic per partial slot and head

struct SimUnit {
  AttnWork w;
  bool part;
};

double unit_cost(const SimUnit& u) {
  return (u.w.kb1 - u.w.kb0) + kUnitOverhead + (u.part ? kPartOverhead : 0.0);
}

// Modelled makespan and mean slot load of `L` (all heads); *last = the list entry whose
// instance finishes last.
void simulate(const std::vector<SimUnit>& L, int heads, int slots, double* makespan, double* mean, int* last) {
  const int64_t n = (int64_t)L.size(), G = n * heads;
  const int64_t per = G >> 3, rem = G & 7;
  double total = 0.0;
  *makespan = 0.0;
  *last = -1;
  std::vector<double> heap;
  for (int64_t x = 0; x < 8; ++x) {
    const int64_t start = x * per + std::min(x, rem), cnt = per + (x < rem ? 1 : 0);
    heap.assign((size_t)slots, 0.0);
    for (int64_t l = start; l < start + cnt; ++l) {
      const int e = (int)(l % n);
      const double c = unit_cost(L[e]);
      std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
      const double t = heap.back() + c;
      heap.back() = t;
      std::push_heap(heap.begin(), heap.end(), std::greater<double>());
      total += c;
      if (t > *makespan) {
        *makespan = t;
        *last = e;
      }
    }
  }
  *mean = total / (8.0 * slots);
}

// Long segments go to 4-wave workgroups of 256 queries, short ones to 1-wave
// workgroups of 64 queries; long units are ordered largest segment first.
void build_lists(const std::vector<Seg>& segs, std::vector<uint8_t>& blob, AttnLists& out,
                 int32_t& max_len, int heads, int n_cu) {
  std::vector<AttnWork> lw, sw;
  out.sq_long = out.sq_short = 0.0;
  std::vector<Seg> order(segs);
  std::stable_sort(order.begin(), order.end(),
                   [](const Seg& a, const Seg& b) { return a.len > b.len; });
  max_len = 0;
  for (const Seg& s : order) {
    max_len = std::max(max_len, s.len);
    const int32_t nkb = (s.len + kAttnKB - 1) / kAttnKB;
    if (s.len > 128) {
      for (int32_t q0 = 0; q0 < s.len; q0 += kAttnQB) lw.push_back({s.start, s.len, q0, 0, nkb, -1, {0, 0}});
      out.sq_long += (double)s.len * s.len;
    } else {
      for (int32_t q0 = 0; q0 < s.len; q0 += 64) sw.push_back({s.start, s.len, q0, 0, nkb, -1, {0, 0}});
      out.sq_short += (double)s.len * s.len;
    }
  }
  out.n_long = (int32_t)lw.size();
  out.n_short = (int32_t)sw.size();
  out.off_long = put(blob, lw);
  out.off_short = put(blob, sw);

  // key splits
  out.n_long_split = out.n_merge = out.n_parts = 0;
  if (lw.empty() || heads <= 0) return;
  const int slots = std::max(1, n_cu / 8) * 2;
  std::vector<SimUnit> L;
  for (const AttnWork& w : lw) L.push_back({w, false});
  double ms0, mean, ms;
  int last;
  simulate(L, heads, slots, &ms0, &mean, &last);
  auto merge_cost = [&](const std::vector<SimUnit>& v) {
    int parts = 0;
    for (const SimUnit& u : v) parts += u.part ? 1 : 0;
    return parts ? kMergeFixed + kMergePerSlot * parts * heads : 0.0;
  };
  std::vector<SimUnit> best = L;
  double best_t = ms0;
  ms = ms0;
  for (int it = 0; it < 128 && ms > 1.03 * mean && last >= 0; ++it) {
    const SimUnit u = L[last];
    const int32_t nb = u.w.kb1 - u.w.kb0;
    if (nb < 2 * kMinPartBlocks) break;
    int32_t parts_of_block = 0;   // parts this query block would have after the split
    for (const SimUnit& v : L)
      if (v.w.seg_start == u.w.seg_start && v.w.q0 == u.w.q0) ++parts_of_block;
    if (parts_of_block + 1 > kAttnMaxParts) break;
    const int32_t mid = u.w.kb0 + nb / 2;
    SimUnit lo = u, hi = u;
    lo.w.kb1 = mid;
    hi.w.kb0 = mid;
    lo.part = hi.part = true;
    L.erase(L.begin() + last);
    L.push_back(lo);
    L.push_back(hi);
    std::stable_sort(L.begin(), L.end(),
                     [](const SimUnit& a, const SimUnit& b) { return unit_cost(a) > unit_cost(b); });
    simulate(L, heads, slots, &ms, &mean, &last);
    const double t = ms + merge_cost(L);
    if (t < best_t) {
      best_t = t;
      best = L;
    }
  }
  if (best_t > 0.97 * ms0) return;   // not worth a merge pass

  // partial slots: the parts of one query block get consecutive slots, in key order
  std::vector<AttnWork> split;
  std::vector<AttnMerge> merges;
  for (const SimUnit& u : best) split.push_back(u.w);
  for (size_t i = 0; i < split.size(); ++i) {
    AttnWork& w = split[i];
    if (!best[i].part || w.part >= 0) continue;
    std::vector<size_t> members;
    for (size_t j = 0; j < split.size(); ++j)
      if (best[j].part && split[j].seg_start == w.seg_start && split[j].q0 == w.q0) members.push_back(j);
    std::sort(members.begin(), members.end(), [&](size_t a, size_t b) { return split[a].kb0 < split[b].kb0; });
    merges.push_back({w.seg_start, w.seg_len, w.q0, out.n_parts, (int32_t)members.size(), {0, 0, 0}});
    for (size_t j : members) split[j].part = out.n_parts++;
  }
  out.n_long_split = (int32_t)split.size();
  out.n_merge = (int32_t)merges.size();
  out.off_long_split = put(blob, split);
  out.off_merge = put(blob, merges);
}

}  // namespace

vit_status build_plan(const vit_ctx* ctx, const int32_t* grid_thw, const int32_t* n_frames,
                      int32_t n_items, vit_plan* p, bool key_splits) {
  const vit_config& c = ctx->cfg;
  p->cfg = c;
  p->head_dim = ctx->head_dim;
  p->mlp_pad = ctx->mlp_pad;
  p->split = ctx->split;
  p->f8 = ctx->f8;
  if (n_items < 0) {
    set_error("n_items must be >= 0 (got %d)", n_items);
    return VIT_E_ARG;
  }
  if (n_items > 0 && (!grid_thw || !n_frames)) {
    set_error("grid_thw and n_frames must not be NULL");
    return VIT_E_ARG;
  }
  p->n_items = n_items;
  p->grid.assign(grid_thw, grid_thw + 3 * (size_t)n_items);
  p->nframes.assign(n_frames, n_frames + (size_t)n_items);

  int64_t n_rows = 0;
  size_t px = 0;
  int32_t max_pos = 1;
  for (int i = 0; i < n_items; ++i) {
    const int32_t t = grid_thw[3 * i], h = grid_thw[3 * i + 1], w = grid_thw[3 * i + 2];
    const int32_t nf = n_frames[i];
    if (t < 1 || h < 2 || w < 2 || (h % kMerge) || (w % kMerge)) {
      set_error("item %d: grid_thw (%d,%d,%d) needs t >= 1 and even h, w >= 2", i, t, h, w);
      return VIT_E_SHAPE;
    }
    if (h > 16384 || w > 16384) {
      set_error("item %d: h, w must be <= 16384 patches", i);
      return VIT_E_SHAPE;
    }
    if (!((nf == 1 && t == 1) || (nf == kTemporal * t))) {
      set_error("item %d: n_frames %d does not match t=%d (1 for an image, 2t for a video)", i, nf,
                t);
      return VIT_E_SHAPE;
    }
    n_rows += (int64_t)t * h * w;
    px += (size_t)nf * (size_t)(kPatch * h) * (size_t)(kPatch * w) * 3;
    max_pos = std::max(max_pos, std::max(h, w));
  }
  if (n_rows > (int64_t)1 << 28) {
    set_error("batch has %lld patches; at most 2^28 are supported", (long long)n_rows);
    return VIT_E_SHAPE;
  }
  p->n_rows = n_rows;
  p->n_units = n_rows / 4;
  p->pixel_bytes = px;
  p->pixel_read_bytes = px;
  p->max_pos = max_pos;
  p->nfreq = ctx->head_dim / 4;

  // ---- device operand extents: the GEMM and attention kernels address each operand with
  // 32-bit buffer offsets, so every one must stay below 2 GiB.  Checked here so that a batch
  // too large for them fails before anything is enqueued.
  {
    const int64_t N = n_rows, d = c.hidden;
    const int64_t S = p->split, mp = p->mlp_pad, hd = p->head_dim, U = n_rows / 4;
    const int64_t N16 = round_up(N, 16), U16 = round_up(U, 16), N32 = round_up(N, 32), U32 = round_up(U, 32);
    const int64_t vt_ld = round_up(N, 8) + 40;
    struct Extent {
      const char* what;
      int64_t bytes;
    } ext[] = {{"normalised patches", N16 * kFeatPad * 2},
               {"norm output", N16 * S * d * 2},
               {"merger input", U16 * 4 * S * d * 2},
               {"attention output", N16 * S * d * 2},
               {"e4m3 attention residual", p->f8 ? N32 * d : 0},
               {"MLP activation", N16 * S * mp * 2},
               {"merger hidden", U16 * 4 * S * d * 2},
               {"e4m3 norm residual", p->f8 ? std::max(N32 * d, U32 * 4 * d) : 0},
               {"e4m3 MLP residual", p->f8 ? std::max(N32 * mp, U32 * 4 * d) : 0},
               {"per-head q or k", N * hd * 2},
               {"per-head V^T", vt_ld * hd * 2}};
    for (const Extent& e : ext)
      if (e.bytes >= ((int64_t)1 << 31)) {
        set_error("batch of %lld patches: the %s operand would take %lld bytes; at most 2^31 - 1 are "
                  "addressable", (long long)N, e.what, (long long)e.bytes);
        return VIT_E_SHAPE;
      }
  }

  // ---- rows in internal order
  const int wu = c.window_px > 0 ? c.window_px / kUnitPx : 0;   // window side in merge units
  std::vector<UnitDesc> units;
  std::vector<int32_t> rowpos, unitdst;
  units.reserve(p->n_units);
  rowpos.reserve(n_rows);
  unitdst.reserve(p->n_units);
  p->row_order.clear();
  p->row_order.reserve(n_rows);
  std::vector<Seg> item_segs, win_segs;
  int64_t px_base = 0, unit_base = 0;
  for (int i = 0; i < n_items; ++i) {
    const int32_t t = grid_thw[3 * i], h = grid_thw[3 * i + 1], w = grid_thw[3 * i + 2];
    const int32_t nf = n_frames[i];
    const int64_t W = (int64_t)kPatch * w, H = (int64_t)kPatch * h;
    const int64_t frame_bytes = H * W * 3;
    if (nf > 1 && frame_bytes > INT32_MAX) {
      // the unit descriptors hold the frame stride as a 32-bit byte count
      set_error("item %d: a %lld x %lld video frame (%lld bytes) exceeds the 2^31-byte frame limit", i,
                (long long)H, (long long)W, (long long)frame_bytes);
      return VIT_E_SHAPE;
    }
    const int32_t uh = h / kMerge, uw = w / kMerge;
    item_segs.push_back({(int32_t)(unit_base * 4), t * h * w});
    for (int32_t ti = 0; ti < t; ++ti) {
      const int64_t slot0 = (nf == 1) ? 0 : (int64_t)kTemporal * ti;
      auto emit = [&](int32_t bh, int32_t bw) {
        UnitDesc u;
        u.px_off = px_base + slot0 * frame_bytes + (int64_t)kUnitPx * bh * W * 3 +
                   (int64_t)kUnitPx * bw * 3;
        u.pitch = (int32_t)(W * 3);
        u.fstride = (nf == 1) ? 0 : (int32_t)frame_bytes;
        units.push_back(u);
        const int64_t orig = unit_base + (int64_t)ti * uh * uw + (int64_t)bh * uw + bw;
        unitdst.push_back((int32_t)orig);
        for (int dh = 0; dh < kMerge; ++dh)
          for (int dw = 0; dw < kMerge; ++dw) {
            rowpos.push_back(((kMerge * bh + dh) << 16) | (kMerge * bw + dw));
            p->row_order.push_back((int32_t)(4 * orig + kMerge * dh + dw));
          }
      };
      if (wu > 0) {
        for (int32_t wy = 0; wy < uh; wy += wu)
          for (int32_t wx = 0; wx < uw; wx += wu) {
            const int32_t start = (int32_t)(units.size() * 4);
            for (int32_t bh = wy; bh < std::min(uh, wy + wu); ++bh)
              for (int32_t bw = wx; bw < std::min(uw, wx + wu); ++bw) emit(bh, bw);
            win_segs.push_back({start, (int32_t)(units.size() * 4) - start});
          }
      } else {
        for (int32_t bh = 0; bh < uh; ++bh)
          for (int32_t bw = 0; bw < uw; ++bw) emit(bh, bw);
      }
    }
    unit_base += (int64_t)t * uh * uw;
    px_base += (int64_t)nf * frame_bytes;
  }

  // ---- 2D RoPE cos/sin cache: [max_pos][nfreq], angle = pos * theta^(-2j / (head_dim/2))
  const int nfreq = p->nfreq;
  const double rd = ctx->head_dim / 2;
  std::vector<float> cs((size_t)max_pos * nfreq), sn((size_t)max_pos * nfreq);
  for (int32_t pos = 0; pos < max_pos; ++pos)
    for (int j = 0; j < nfreq; ++j) {
      const double a = (double)pos * std::pow((double)c.rope_theta, -2.0 * j / rd);
      cs[(size_t)pos * nfreq + j] = (float)std::cos(a);
      sn[(size_t)pos * nfreq + j] = (float)std::sin(a);
    }

  std::vector<uint8_t>& blob = p->meta;
  blob.clear();
  p->off_dims = put(blob, std::vector<RunDims>(1, RunDims{}));   // filled in below
  p->off_units = put(blob, units);
  p->off_rowpos = put(blob, rowpos);
  p->off_unitdst = put(blob, unitdst);
  p->off_cos = put(blob, cs);
  p->off_sin = put(blob, sn);
  const int n_cu = ctx->n_cu > 0 ? ctx->n_cu : 256;
  const int split_heads = key_splits ? c.heads : 0;   // 0: no key splits
  build_lists(item_segs, blob, p->full, p->max_seg_full, split_heads, n_cu);
  if (wu > 0) build_lists(win_segs, blob, p->win, p->max_seg_win, split_heads, n_cu);
  blob.resize(round_up((int64_t)blob.size(), 256));
  RunDims dims{};
  dims.n_rows = (int32_t)n_rows;
  dims.n_units = (int32_t)p->n_units;
  dims.full_long = p->full.n_long;
  dims.full_short = p->full.n_short;
  dims.win_long = p->win.n_long;
  dims.win_short = p->win.n_short;
  std::memcpy(blob.data() + p->off_dims, &dims, sizeof dims);

  // ---- workspace layout
  const int64_t N = n_rows, d = c.hidden;
  size_t off = blob.size();
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up((int64_t)(off + bytes), 256);
    return o;
  };
  // GEMM operands (X, H, O, F) are blocked: rows padded to whole 16-row groups, for the
  // patch rows (N) and for the merger's view of them (N / 4 rows of 4 patch rows each)
  const int64_t Np = round_up(N, 16), Up = round_up(N / 4, 16);
  const int64_t S = p->split;
  p->off_x = take((size_t)Np * kFeatPad * 2);
  p->off_r = take((size_t)N * d * 4);
  p->off_h = take((size_t)std::max(Np * S * d, Up * 4 * S * d) * 2);
  p->off_q = take((size_t)N * d * 2);
  p->off_k = take((size_t)N * d * 2);
  // V^T rows: a pitch that is a multiple of 8 tokens, with at least 40 columns past the last
  // token that are zeroed every forward.  A key block's load reaches up to 31 tokens past a
  // segment's last key (keys that get probability 0); those columns must hold finite values,
  // since 0 * NaN is NaN inside the MFMA, and must stay inside the row.
  p->vt_ld = round_up(N, 8) + 40;
  p->off_vt = take((size_t)p->vt_ld * d * 2);
  p->off_o = take((size_t)Np * S * d * 2);
  p->off_f = take((size_t)std::max(Np * S * p->mlp_pad, Up * 4 * S * d) * 2);
  if (p->f8) {   // e4m3 residuals of H and F: rows padded to whole 32-row groups
    const int64_t N32 = round_up(N, 32), U32 = round_up(N / 4, 32);
    p->off_h8 = take((size_t)std::max(N32 * d, U32 * 4 * d));
    p->off_f8 = take((size_t)std::max(N32 * p->mlp_pad, U32 * 4 * d));
    p->off_o8 = take((size_t)N32 * d);
  }
  const int32_t n_parts = std::max(p->full.n_parts, p->win.n_parts);
  p->off_part = n_parts > 0 ? take((size_t)c.heads * n_parts * (p->head_dim + 2) * kAttnQB * 4) : 0;
  p->off_pix = take(px);
  p->off_out = take((size_t)p->n_units * c.out_dim * 4);
  p->ws_bytes = off;
  return VIT_OK;
}

}  // namespace vitmi
