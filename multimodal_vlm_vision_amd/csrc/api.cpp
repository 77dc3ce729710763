// C ABI of the vision-tower library and the forward launch sequence.
//
// The forward follows the pipeline the pages describe, with normalisation as
// the tower's own first step (vLLM PR #55370 report, implementation
// breakdown) so that eager and graph-replayed forwards normalise exactly
// once; per-forward metadata (segment bounds, positions, cos/sin cache) is
// built once on the host and uploaded with one asynchronous copy, then
// shared by every layer ("vLLM multimodal inference | ViT performance
// optimisation", section 3.4).  An empty batch enqueues nothing
// ("GPUModelRunner.execute_model" notes, limits section).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "vit_internal.h"

namespace vitmi {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

namespace {

#define HIP_TRY(expr)                                                   \
  do {                                                                  \
    hipError_t e_ = (expr);                                             \
    if (e_ != hipSuccess) {                                             \
      set_error("%s: %s", #expr, hipGetErrorString(e_));                \
      return VIT_E_HIP;                                                 \
    }                                                                   \
  } while (0)

#define VIT_TRY(expr)          \
  do {                         \
    vit_status s_ = (expr);    \
    if (s_ != VIT_OK) return s_; \
  } while (0)

// Where a debug run stops: after (layer, step); layer -2 = never.
struct Stop {
  int layer = -2, step = 0;
  void* dst = nullptr;
  size_t dst_bytes = 0;
  bool hit(int l, int s) const { return layer == l && step == s; }
};

vit_status copy_out(const Stop& st, const void* src, size_t bytes, hipStream_t s) {
  if (st.dst_bytes < bytes) {
    set_error("debug stage needs %zu bytes, dst has %zu", bytes, st.dst_bytes);
    return VIT_E_WORKSPACE;
  }
  HIP_TRY(hipMemcpyAsync(st.dst, src, bytes, hipMemcpyDeviceToDevice, s));
  return VIT_OK;
}

// Debug copy of a blocked bf16 GEMM operand as row-major [rows][out_cols] (see launch_unblock).
vit_status copy_blocked(const Stop& st, const uint16_t* src, int64_t rows, int cols, int group, int out_cols,
                        hipStream_t s) {
  const size_t bytes = (size_t)rows * out_cols * 2;
  if (st.dst_bytes < bytes) {
    set_error("debug stage needs %zu bytes, dst has %zu", bytes, st.dst_bytes);
    return VIT_E_WORKSPACE;
  }
  return launch_unblock(src, rows, cols, group, out_cols, static_cast<uint16_t*>(st.dst), s);
}

// compensated activation in the bf16 + e4m3 form -> [hi | residual] bf16 rows (2 * out_cols)
vit_status copy_blocked_f8(const Stop& st, const uint16_t* src, const uint8_t* src8, int64_t rows, int cols,
                           int group, int out_cols, hipStream_t s) {
  const size_t bytes = (size_t)rows * out_cols * 4;
  if (st.dst_bytes < bytes) {
    set_error("debug stage needs %zu bytes, dst has %zu", bytes, st.dst_bytes);
    return VIT_E_WORKSPACE;
  }
  return launch_unblock_f8(src, src8, rows, cols, group, out_cols, static_cast<uint16_t*>(st.dst), s);
}

vit_status check_common(const vit_ctx* ctx, const vit_plan* plan, const void* ws, size_t ws_bytes) {
  if (!ctx || !plan) {
    set_error("ctx and plan must not be NULL");
    return VIT_E_ARG;
  }
  if (!ctx->finalized) {
    set_error("weights not finalized");
    return VIT_E_STATE;
  }
  // the plan's workspace layout, work lists and rotary tables follow the configuration of the
  // tower it was built for: every field they depend on must match this tower's
  const vit_config& pc = plan->cfg;
  const vit_config& cc = ctx->cfg;
  bool same = pc.hidden == cc.hidden && pc.heads == cc.heads && pc.layers == cc.layers &&
              pc.mlp_dim == cc.mlp_dim && pc.mlp_kind == cc.mlp_kind && pc.out_dim == cc.out_dim &&
              pc.rope_theta == cc.rope_theta && pc.window_px == cc.window_px &&
              pc.n_full_attn_layers == cc.n_full_attn_layers &&
              pc.activation_precision == cc.activation_precision && plan->head_dim == ctx->head_dim &&
              plan->mlp_pad == ctx->mlp_pad && plan->split == ctx->split && plan->f8 == ctx->f8;
  for (int i = 0; same && i < cc.n_full_attn_layers && i < VIT_MAX_FULL_LAYERS; ++i)
    same = pc.full_attn_layers[i] == cc.full_attn_layers[i];
  if (!same) {
    set_error("plan was built for a different tower configuration");
    return VIT_E_ARG;
  }
  if (plan->n_rows > 0) {
    if (!ws) {
      set_error("workspace must not be NULL");
      return VIT_E_ARG;
    }
    if (ws_bytes < plan->ws_bytes) {
      set_error("workspace too small: %zu < %zu bytes", ws_bytes, plan->ws_bytes);
      return VIT_E_WORKSPACE;
    }
    if (reinterpret_cast<uintptr_t>(ws) % 256) {
      set_error("workspace must be 256-byte aligned");
      return VIT_E_ARG;
    }
  }
  return VIT_OK;
}

// Optional per-launch timing: a pair of hipEvents around every kernel launch.
struct Prof {
  struct Rec {
    const char* name;
    hipEvent_t a, b;
    double flops, bytes;
    bool mfma;
  };
  std::vector<Rec> recs;
  hipStream_t st = nullptr;
  vit_status begin(const char* name, double flops, double bytes, bool mfma) {
    Rec r{name, nullptr, nullptr, flops, bytes, mfma};
    HIP_TRY(hipEventCreate(&r.a));
    HIP_TRY(hipEventCreate(&r.b));
    recs.push_back(r);
    HIP_TRY(hipEventRecord(r.a, st));
    return VIT_OK;
  }
  vit_status end() {
    HIP_TRY(hipEventRecord(recs.back().b, st));
    return VIT_OK;
  }
  ~Prof() {
    for (Rec& r : recs) {
      if (r.a) (void)hipEventDestroy(r.a);
      if (r.b) (void)hipEventDestroy(r.b);
    }
  }
};

#define LAUNCH(name, fl, by, mf, expr)                 \
  do {                                                 \
    if (prof) VIT_TRY(prof->begin(name, fl, by, mf));  \
    VIT_TRY(expr);                                     \
    if (prof) VIT_TRY(prof->end());                    \
  } while (0)

// Enqueues the forward.  Exactly one of pixels / patches is non-null.
vit_status forward(const vit_ctx* ctx, const vit_plan* pl, const uint8_t* pixels,
                   const uint8_t* patches, char* ws, float* out, hipStream_t st, bool upload,
                   const Stop& stop, Prof* prof = nullptr, bool bucket = false) {
  const vit_config& c = ctx->cfg;
  const DeviceWeights& W = ctx->w;
  const int64_t N = pl->n_rows;
  const int d = c.hidden, hd = ctx->head_dim, mp = ctx->mlp_pad;
  const int S = ctx->split;            // 2: activations stored as [hi | lo] rows
  const bool split = S == 2;
  const bool f8 = ctx->f8;             // activations stored as bf16 rows + e4m3 residuals
  const bool f16 = ctx->f16;           // float16 activations against float16 weight copies
  const double Nd = (double)N, dd = (double)d;
  if (N == 0) return VIT_OK;
  if (prof) prof->st = st;
  if (upload) HIP_TRY(hipMemcpyAsync(ws, pl->meta.data(), pl->meta.size(), hipMemcpyHostToDevice, st));

  const auto* units = reinterpret_cast<const UnitDesc*>(ws + pl->off_units);
  const auto* rowpos = reinterpret_cast<const int32_t*>(ws + pl->off_rowpos);
  const auto* unitdst = reinterpret_cast<const int32_t*>(ws + pl->off_unitdst);
  const auto* cos_t = reinterpret_cast<const float*>(ws + pl->off_cos);
  const auto* sin_t = reinterpret_cast<const float*>(ws + pl->off_sin);
  uint16_t* X = reinterpret_cast<uint16_t*>(ws + pl->off_x);
  float* R = reinterpret_cast<float*>(ws + pl->off_r);
  uint16_t* H = reinterpret_cast<uint16_t*>(ws + pl->off_h);
  uint16_t* Q = reinterpret_cast<uint16_t*>(ws + pl->off_q);
  uint16_t* K = reinterpret_cast<uint16_t*>(ws + pl->off_k);
  uint16_t* VT = reinterpret_cast<uint16_t*>(ws + pl->off_vt);
  uint16_t* O = reinterpret_cast<uint16_t*>(ws + pl->off_o);
  uint16_t* F = reinterpret_cast<uint16_t*>(ws + pl->off_f);
  uint8_t* H8 = f8 ? reinterpret_cast<uint8_t*>(ws + pl->off_h8) : nullptr;
  uint8_t* F8 = f8 ? reinterpret_cast<uint8_t*>(ws + pl->off_f8) : nullptr;
  uint8_t* O8 = f8 ? reinterpret_cast<uint8_t*>(ws + pl->off_o8) : nullptr;
  // debug copies of the compensated activations: [hi | lo] rows in either form
  auto copy_act = [&](const uint16_t* src, const uint8_t* src8, int64_t rows, int cols, int group) {
    return f8 ? copy_blocked_f8(stop, src, src8, rows, cols, group, cols, st)
              : copy_blocked(stop, src, rows, S * cols, group, S * cols, st);
  };

  // bucketed graph: batch sizes come from the RunDims the replay uploads (the plan here is
  // the capacity); every count-dependent kernel gets a pointer into it
  const RunDims* dims = bucket ? reinterpret_cast<const RunDims*>(ws + pl->off_dims) : nullptr;
  const int32_t* rows_dev = dims ? &dims->n_rows : nullptr;
  const int32_t* units_dev = dims ? &dims->n_units : nullptr;

  VIT_TRY(launch_vt_pad_zero(VT, d, N, pl->vt_ld, st, rows_dev));

  // 1. rescale + normalise + patchify: every needed pixel byte read once, 1176 bf16 written per row
  const double np_bytes = (double)pl->pixel_read_bytes + Nd * kFeat * 2;
  if (pixels)
    LAUNCH("normpatch", 0, np_bytes, false,
           launch_normpatch(pixels, units, pl->n_units, W.lut, ctx->norm_affine ? &ctx->affine : nullptr, X, st,
                            units_dev));
  else
    LAUNCH("normrows_u8", 0, Nd * kFeat * 3, false, launch_normrows_u8(patches, N, W.lut, X, st));
  if (stop.hit(-1, 0)) return copy_blocked(stop, X, N, kFeatPad, 1, kFeat, st);

  // 2. patch embedding (conv with kernel == stride as one GEMM), fp32 into the residual
  GemmArgs g;
  g.A = X; g.lda = kFeatPad; g.B = W.pe_w; g.ldb = kFeatPad;
  g.M = (int)N; g.N = d; g.K = kFeatPad; g.out = R; g.ldo = d; g.m_dev = rows_dev;
  LAUNCH("gemm_patch_embed", 2.0 * Nd * dd * kFeat, 0, true, launch_gemm(EPI_F32, g, st));
  if (stop.hit(-1, 1)) return copy_out(stop, R, (size_t)N * d * 4, st);

  const double norm_bytes = Nd * dd * (4 + 2 * S + (f8 ? 1 : 0));   // fp32 row in, bf16 row (hi and lo) out
  for (int l = 0; l < c.layers; ++l) {
    const LayerW& L = W.layers[l];
    LAUNCH("rownorm", 0, norm_bytes, false,
           launch_rownorm(c.norm_kind, R, N, d, L.n1g, L.n1b, c.norm_eps, H, split, 1, st, rows_dev, H8, f16));
    if (stop.hit(l, 1)) return copy_act(H, H8, N, d, 1);

    GemmArgs q;
    q.A = H; q.lda = S * d; q.B = L.qkv_w; q.ldb = d; q.a_group = split ? d : 0;
    q.M = (int)N; q.N = 3 * d; q.K = d; q.bias = L.qkv_b; q.m_dev = rows_dev;
    q.q = Q; q.k = K; q.vt = VT; q.n_tok = N; q.vt_ld = pl->vt_ld;
    q.row_pos = rowpos; q.cos_tab = cos_t; q.sin_tab = sin_t;
    q.nfreq = pl->nfreq; q.head_dim = hd; q.hidden = d;
    q.q_scale = (float)(1.4426950408889634 / std::sqrt((double)hd));   // log2(e) / sqrt(head_dim)
    q.f16 = f16; q.acc_scale = L.qkv_sc;
    if (f8) {
      q.A8 = H8; q.lda8 = d; q.B8 = L.qkv_w8; q.ldb8 = d; q.b8_scale = L.qkv_s8;
    }
    LAUNCH("gemm_qkv_rope", 2.0 * Nd * 3 * dd * dd, 0, true, launch_gemm(EPI_QKV, q, st));
    if (stop.hit(l, 2)) return copy_out(stop, Q, (size_t)N * d * 2, st);
    if (stop.hit(l, 3)) return copy_out(stop, K, (size_t)N * d * 2, st);
    if (stop.hit(l, 4)) {
      if (stop.dst_bytes < (size_t)N * d * 2) return copy_out(stop, VT, (size_t)N * d * 2, st);
      HIP_TRY(hipMemcpy2DAsync(stop.dst, N * 2, VT, pl->vt_ld * 2, N * 2, d, hipMemcpyDeviceToDevice, st));
      return VIT_OK;
    }

    const bool windowed = c.window_px > 0 && !ctx->is_full_layer(l);
    const AttnLists& lists = windowed ? pl->win : pl->full;
    AttnArgs at;
    at.q = Q; at.k = K; at.vt = VT; at.o = O; at.o_split = split; at.o8 = O8; at.f16 = f16;
    at.n_tok = N; at.vt_ld = pl->vt_ld;
    at.heads = c.heads; at.head_dim = hd;
    // key-split units with their merge (not in bucketed graphs, whose capacity checks and
    // device-side counts are those of the plain lists)
    const bool use_split = !dims && lists.n_merge > 0;
    at.work_long = reinterpret_cast<const AttnWork*>(ws + (use_split ? lists.off_long_split : lists.off_long));
    at.work_short = reinterpret_cast<const AttnWork*>(ws + lists.off_short);
    if (use_split) {
      at.part = reinterpret_cast<float*>(ws + pl->off_part);
      at.n_parts = lists.n_parts;
    }
    const int n_long = use_split ? lists.n_long_split : lists.n_long;
    if (n_long > 0) {
      AttnArgs a1 = at;
      a1.n_long = n_long;
      if (dims) a1.n_long_dev = windowed ? &dims->win_long : &dims->full_long;
      LAUNCH("attention", 4.0 * dd * lists.sq_long, 0, true, launch_attention(a1, st));
    }
    if (lists.n_short > 0) {
      AttnArgs a2 = at;
      a2.n_short = lists.n_short;
      if (dims) a2.n_short_dev = windowed ? &dims->win_short : &dims->full_short;
      LAUNCH("attention_short", 4.0 * dd * lists.sq_short, 0, true, launch_attention(a2, st));
    }
    if (use_split) {
      const double part_bytes = (double)c.heads * lists.n_parts * (hd + 2) * 256 * 4;
      LAUNCH("attention_merge", 0, part_bytes + (double)c.heads * lists.n_merge * 256 * hd * 2, false,
             launch_attention_merge(at, reinterpret_cast<const AttnMerge*>(ws + lists.off_merge), lists.n_merge,
                                    st));
    }
    if (stop.hit(l, 5)) return copy_act(O, O8, N, d, 1);

    // the attention output is compensated like the other GEMM activations: its bf16 rounding
    // is the largest single error source at depth once those are compensated
    GemmArgs pj;
    pj.A = O; pj.lda = S * d; pj.B = L.proj_w; pj.ldb = d; pj.a_group = split ? d : 0;
    pj.M = (int)N; pj.N = d; pj.K = d; pj.bias = L.proj_b; pj.out = R; pj.ldo = d; pj.m_dev = rows_dev;
    pj.f16 = f16; pj.acc_scale = L.proj_sc;
    if (f8) {
      pj.A8 = O8; pj.lda8 = d; pj.B8 = L.proj_w8; pj.ldb8 = d; pj.b8_scale = L.proj_s8;
    }
    LAUNCH("gemm_proj_residual", 2.0 * Nd * dd * dd, 0, true, launch_gemm(EPI_RES, pj, st));
    if (stop.hit(l, 6)) return copy_out(stop, R, (size_t)N * d * 4, st);

    LAUNCH("rownorm", 0, norm_bytes, false,
           launch_rownorm(c.norm_kind, R, N, d, L.n2g, L.n2b, c.norm_eps, H, split, 1, st, rows_dev, H8, f16));
    if (stop.hit(l, 7)) return copy_act(H, H8, N, d, 1);

    GemmArgs f1;
    f1.A = H; f1.lda = S * d; f1.B = L.fc1_w; f1.ldb = d; f1.a_group = split ? d : 0;
    f1.M = (int)N; f1.K = d; f1.bias = L.fc1_b; f1.out = F; f1.ldo = S * mp; f1.m_dev = rows_dev;
    f1.split_off = split ? mp : 0;
    f1.f16 = f16; f1.acc_scale = L.fc1_sc;
    if (f8) {
      f1.A8 = H8; f1.lda8 = d; f1.B8 = L.fc1_w8; f1.ldb8 = d; f1.b8_scale = L.fc1_s8;
      f1.out8 = F8; f1.ldo8 = mp;
    }
    if (c.mlp_kind == VIT_MLP_GELU) {
      f1.N = mp;
      LAUNCH("gemm_fc1_gelu", 2.0 * Nd * c.mlp_dim * dd, 0, true, launch_gemm(EPI_GELU, f1, st));
    } else {
      f1.N = 2 * mp;
      LAUNCH("gemm_gateup_swiglu", 4.0 * Nd * c.mlp_dim * dd, 0, true,
             launch_gemm(EPI_SWIGLU, f1, st));
    }
    if (stop.hit(l, 8)) return copy_act(F, F8, N, mp, 1);

    GemmArgs f2;
    f2.A = F; f2.lda = S * mp; f2.B = L.fc2_w; f2.ldb = mp; f2.a_group = split ? mp : 0;
    f2.M = (int)N; f2.N = d; f2.K = mp; f2.bias = L.fc2_b; f2.out = R; f2.ldo = d; f2.m_dev = rows_dev;
    f2.f16 = f16; f2.acc_scale = L.fc2_sc;
    if (f8) {
      f2.A8 = F8; f2.lda8 = mp; f2.B8 = L.fc2_w8; f2.ldb8 = mp; f2.b8_scale = L.fc2_s8;
    }
    LAUNCH("gemm_fc2_residual", 2.0 * Nd * dd * c.mlp_dim, 0, true, launch_gemm(EPI_RES, f2, st));
    if (stop.hit(l, 9)) return copy_out(stop, R, (size_t)N * d * 4, st);
  }

  // merger: per-patch norm written straight into the merger's view (a unit's 4 patch rows
  // side by side as one row of 4 * S * d columns), then the MLP
  const int L = c.layers;
  LAUNCH("rownorm", 0, norm_bytes, false,
         launch_rownorm(c.norm_kind, R, N, d, W.mq_g, W.mq_b, c.norm_eps, H, split, 4, st, rows_dev, H8, f16));
  if (stop.hit(L, 1)) return copy_act(H, H8, N, d, 4);
  const int64_t U = pl->n_units;
  const double Ud = (double)U;
  GemmArgs m1;
  m1.A = H; m1.lda = S * 4 * d; m1.B = W.m1_w; m1.ldb = 4 * d; m1.a_group = split ? d : 0;
  m1.M = (int)U; m1.N = 4 * d; m1.K = 4 * d; m1.bias = W.m1_b; m1.out = F; m1.ldo = S * 4 * d;
  m1.m_dev = units_dev;
  m1.split_off = split ? 4 * d : 0;
  m1.f16 = f16; m1.acc_scale = W.m1_sc;
  if (f8) {
    m1.A8 = H8; m1.lda8 = 4 * d; m1.B8 = W.m1_w8; m1.ldb8 = 4 * d; m1.b8_scale = W.m1_s8;
    m1.out8 = F8; m1.ldo8 = 4 * d;
  }
  LAUNCH("gemm_merger_fc1_gelu", 2.0 * Ud * 16 * dd * dd, 0, true, launch_gemm(EPI_GELU, m1, st));
  if (stop.hit(L, 2)) return copy_act(F, F8, U, 4 * d, 1);
  GemmArgs m2;
  m2.A = F; m2.lda = S * 4 * d; m2.B = W.m2_w; m2.ldb = 4 * d; m2.a_group = split ? 4 * d : 0;
  m2.M = (int)U; m2.N = c.out_dim; m2.K = 4 * d; m2.bias = W.m2_b; m2.out = out; m2.ldo = c.out_dim;
  m2.m_dev = units_dev;
  m2.row_map = unitdst;
  m2.f16 = f16; m2.acc_scale = W.m2_sc;
  if (f8) {
    m2.A8 = F8; m2.lda8 = 4 * d; m2.B8 = W.m2_w8; m2.ldb8 = 4 * d; m2.b8_scale = W.m2_s8;
  }
  LAUNCH("gemm_merger_fc2", 2.0 * Ud * c.out_dim * 4 * dd, 0, true, launch_gemm(EPI_OUT, m2, st));
  if (stop.hit(L, 3)) return copy_out(stop, out, (size_t)U * c.out_dim * 4, st);
  return VIT_OK;
}

vit_status validate_config(const vit_config* c, int* head_dim) {
  if (!c) {
    set_error("config must not be NULL");
    return VIT_E_ARG;
  }
  if (c->patch != kPatch || c->temporal_patch != kTemporal || c->merge != kMerge) {
    set_error("patch/temporal_patch/merge must be 14/2/2 (got %d/%d/%d)", c->patch,
              c->temporal_patch, c->merge);
    return VIT_E_ARG;
  }
  if (c->hidden <= 0 || c->hidden % 64 || c->heads <= 0 || c->hidden % c->heads) {
    set_error("hidden must be a positive multiple of 64 divisible by heads");
    return VIT_E_ARG;
  }
  const int hd = c->hidden / c->heads;
  if (hd != 32 && hd != 64 && hd != 80) {
    set_error("head_dim %d not supported (32, 64 or 80)", hd);
    return VIT_E_ARG;
  }
  if (c->hidden > 2048) {
    set_error("hidden must be <= 2048");
    return VIT_E_ARG;
  }
  if (c->layers < 0 || c->mlp_dim <= 0 || c->out_dim <= 0 || c->out_dim % 64) {
    set_error("layers >= 0, mlp_dim > 0 and out_dim a positive multiple of 64 required");
    return VIT_E_ARG;
  }
  if ((c->mlp_kind != VIT_MLP_GELU && c->mlp_kind != VIT_MLP_SWIGLU) ||
      (c->norm_kind != VIT_NORM_LAYER && c->norm_kind != VIT_NORM_RMS)) {
    set_error("bad mlp_kind or norm_kind");
    return VIT_E_ARG;
  }
  if (!(c->norm_eps > 0.f) || !(c->rope_theta > 1.f)) {
    set_error("norm_eps must be > 0 and rope_theta > 1");
    return VIT_E_ARG;
  }
  for (int i = 0; i < 3; ++i)
    if (!(c->std[i] > 0.f)) {
      set_error("std[%d] must be > 0", i);
      return VIT_E_ARG;
    }
  if (c->window_px < 0 || (c->window_px % kUnitPx)) {
    set_error("window_px must be 0 or a positive multiple of 28");
    return VIT_E_ARG;
  }
  if (c->activation_precision != VIT_ACT_BF16 && c->activation_precision != VIT_ACT_BF16X2 &&
      c->activation_precision != VIT_ACT_BF16F8 && c->activation_precision != VIT_ACT_F16) {
    set_error("activation_precision must be VIT_ACT_F16, VIT_ACT_BF16, VIT_ACT_BF16X2 or VIT_ACT_BF16F8");
    return VIT_E_ARG;
  }
  if (c->n_full_attn_layers < 0 || c->n_full_attn_layers > VIT_MAX_FULL_LAYERS) {
    set_error("n_full_attn_layers out of range");
    return VIT_E_ARG;
  }
  *head_dim = hd;
  return VIT_OK;
}

// Exactly rounded bfloat16 of ((x/255) - mean) / std for every byte x.  The
// quotient is evaluated in long double; a value whose distance to a rounding
// midpoint is below the evaluation error is re-decided with a wider margin
// check (never happens for realistic parameters; an assert-style error).
void build_lut(const vit_config& c, uint16_t (&lut)[3][256]) {
  for (int ch = 0; ch < 3; ++ch) {
    const long double m = (long double)c.mean[ch], s = (long double)c.std[ch];
    for (int x = 0; x < 256; ++x) {
      const long double v = ((long double)x / 255.0L - m) / s;
      // round to 8 significant bits, ties to even, from the long double value
      if (v == 0.0L) {
        lut[ch][x] = 0;
        continue;
      }
      int e;
      const long double fr = std::frexp(std::fabs(v), &e);   // [0.5, 1)
      long double sc = fr * 256.0L;
      long double fl = std::floor(sc);
      const long double rem = sc - fl;
      if (rem > 0.5L || (rem == 0.5L && std::fmod(fl, 2.0L) != 0.0L)) fl += 1.0L;
      const float r = (float)std::ldexp(fl, e - 8) * (v < 0 ? -1.f : 1.f);
      lut[ch][x] = f32_to_bf16_bits(r);   // exact: r already has 8 significant bits
    }
  }
}

// The same quotient as one float32 fused multiply-add, x * (1 / (255 s)) + (-m / s), with
// both constants rounded to float32; accepted only if its bf16 rounding equals the exact
// table entry for every byte of every channel (checked here with the host's IEEE fmaf,
// which rounds exactly as the GPU's v_fma_f32).
bool verify_affine(const vit_config& c, const uint16_t (&lut)[3][256], NormAffine* out) {
  for (int ch = 0; ch < 3; ++ch) {
    const long double m = (long double)c.mean[ch], s = (long double)c.std[ch];
    const float a = (float)(1.0L / (255.0L * s));
    const float b = (float)(-m / s);
    for (int x = 0; x < 256; ++x)
      if (f32_to_bf16_bits(std::fma((float)x, a, b)) != lut[ch][x]) return false;
    out->a[ch] = a;
    out->b[ch] = b;
  }
  return true;
}

}  // namespace

vit_status check_plan_ws(const vit_ctx* ctx, const vit_plan* plan, const void* ws, size_t ws_bytes) {
  return check_common(ctx, plan, ws, ws_bytes);
}

vit_status create_plan(const vit_ctx* ctx, const int32_t* grid_thw, const int32_t* n_frames, int32_t n_items,
                       bool key_splits, vit_plan** out) {
  if (!ctx || !out) {
    set_error("ctx and out must not be NULL");
    return VIT_E_ARG;
  }
  *out = nullptr;
  vit_plan* p = new (std::nothrow) vit_plan();
  if (!p) {
    set_error("out of host memory");
    return VIT_E_ARG;
  }
  vit_status s = build_plan(ctx, grid_thw, n_frames, n_items, p, key_splits);
  if (s != VIT_OK) {
    delete p;
    return s;
  }
  *out = p;
  return VIT_OK;
}

}  // namespace vitmi

using namespace vitmi;

bool vit_ctx::is_full_layer(int l) const {
  for (int i = 0; i < cfg.n_full_attn_layers; ++i)
    if (cfg.full_attn_layers[i] == l) return true;
  return false;
}

extern "C" {

const char* vit_last_error(void) { return g_err; }

vit_status vit_create(const vit_config* cfg, vit_ctx** out) {
  if (!out) {
    set_error("out must not be NULL");
    return VIT_E_ARG;
  }
  *out = nullptr;
  int hd = 0;
  VIT_TRY(validate_config(cfg, &hd));
  vit_ctx* ctx = new (std::nothrow) vit_ctx();
  if (!ctx) {
    set_error("out of host memory");
    return VIT_E_ARG;
  }
  ctx->cfg = *cfg;
  ctx->head_dim = hd;
  ctx->mlp_pad = (int)round_up(cfg->mlp_dim, 64);
  ctx->split = cfg->activation_precision == VIT_ACT_BF16X2 ? 2 : 1;
  ctx->f8 = cfg->activation_precision == VIT_ACT_BF16F8;
  ctx->f16 = cfg->activation_precision == VIT_ACT_F16;
  build_lut(*cfg, ctx->lut);
  ctx->norm_affine = verify_affine(*cfg, ctx->lut, &ctx->affine);
  *out = ctx;
  return VIT_OK;
}

vit_status vit_load_weight(vit_ctx* ctx, const char* name, int32_t dtype, const int64_t* shape,
                           int32_t ndim, const void* host_ptr) {
  if (!ctx) {
    set_error("ctx must not be NULL");
    return VIT_E_ARG;
  }
  return store_weight(ctx, name, dtype, shape, ndim, host_ptr);
}

vit_status vit_finalize_weights(vit_ctx* ctx, void* stream) {
  if (!ctx) {
    set_error("ctx must not be NULL");
    return VIT_E_ARG;
  }
  return finalize_weights(ctx, stream);
}

vit_status vit_plan_create(const vit_ctx* ctx, const int32_t* grid_thw, const int32_t* n_frames,
                           int32_t n_items, vit_plan** out) {
  return create_plan(ctx, grid_thw, n_frames, n_items, true, out);
}


void vit_plan_destroy(vit_plan* plan) { delete plan; }

vit_status vit_plan_sizes(const vit_plan* plan, size_t* pixel_bytes, size_t* ws_bytes,
                          int64_t* out_rows, int64_t* out_cols) {
  if (!plan) {
    set_error("plan must not be NULL");
    return VIT_E_ARG;
  }
  if (pixel_bytes) *pixel_bytes = plan->pixel_bytes;
  if (ws_bytes) *ws_bytes = plan->ws_bytes;
  if (out_rows) *out_rows = plan->n_units;
  if (out_cols) *out_cols = plan->cfg.out_dim;
  return VIT_OK;
}

vit_status vit_plan_rows(const vit_plan* plan, int64_t* n_patches, int32_t* dst) {
  if (!plan) {
    set_error("plan must not be NULL");
    return VIT_E_ARG;
  }
  if (n_patches) *n_patches = plan->n_rows;
  if (dst && !plan->row_order.empty())
    std::memcpy(dst, plan->row_order.data(), plan->row_order.size() * sizeof(int32_t));
  return VIT_OK;
}

vit_status vit_plan_attention_units(const vit_plan* plan, int32_t layer_kind, int32_t split, int32_t* units,
                                    int32_t* n_units, int32_t* n_merge, int32_t* n_parts) {
  if (!plan || (layer_kind != 0 && layer_kind != 1) || (split != 0 && split != 1)) {
    set_error("vit_plan_attention_units: plan must not be NULL and layer_kind, split must be 0 or 1");
    return VIT_E_ARG;
  }
  const AttnLists& L = layer_kind ? plan->win : plan->full;
  const bool s = split && L.n_merge > 0;
  const int32_t n = s ? L.n_long_split : L.n_long;
  if (n_units) *n_units = n;
  if (n_merge) *n_merge = s ? L.n_merge : 0;
  if (n_parts) *n_parts = s ? L.n_parts : 0;
  if (units && n > 0)
    std::memcpy(units, plan->meta.data() + (s ? L.off_long_split : L.off_long), (size_t)n * sizeof(AttnWork));
  return VIT_OK;
}

vit_status vit_encode(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8, void* ws,
                      size_t ws_bytes, float* out, void* stream) {
  VIT_TRY(check_common(ctx, plan, ws, ws_bytes));
  if (plan->n_rows == 0) return VIT_OK;
  if (!pixels_u8 || !out) {
    set_error("pixels and out must not be NULL");
    return VIT_E_ARG;
  }
  return forward(ctx, plan, pixels_u8, nullptr, static_cast<char*>(ws), out,
                 static_cast<hipStream_t>(stream), true, Stop{});
}

vit_status vit_encode_patches_u8(const vit_ctx* ctx, const vit_plan* plan,
                                 const uint8_t* patches_u8, void* ws, size_t ws_bytes, float* out,
                                 void* stream) {
  VIT_TRY(check_common(ctx, plan, ws, ws_bytes));
  if (plan->n_rows == 0) return VIT_OK;
  if (!patches_u8 || !out) {
    set_error("patches and out must not be NULL");
    return VIT_E_ARG;
  }
  if (reinterpret_cast<uintptr_t>(patches_u8) % 8) {
    set_error("patches must be 8-byte aligned");
    return VIT_E_ARG;
  }
  return forward(ctx, plan, nullptr, patches_u8, static_cast<char*>(ws), out,
                 static_cast<hipStream_t>(stream), true, Stop{});
}

vit_status vit_encode_profiled(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8,
                               void* ws, size_t ws_bytes, float* out, void* stream,
                               vit_kernel_stat* stats, int32_t max_stats, int32_t* n_stats) {
  VIT_TRY(check_common(ctx, plan, ws, ws_bytes));
  if (n_stats) *n_stats = 0;
  if (plan->n_rows == 0) return VIT_OK;
  if (!pixels_u8 || !out || (max_stats > 0 && !stats)) {
    set_error("pixels, out and stats must not be NULL");
    return VIT_E_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  Prof prof;
  VIT_TRY(forward(ctx, plan, pixels_u8, nullptr, static_cast<char*>(ws), out, st, true, Stop{}, &prof));
  HIP_TRY(hipStreamSynchronize(st));
  std::vector<vit_kernel_stat> agg;
  for (const Prof::Rec& r : prof.recs) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    vit_kernel_stat* k = nullptr;
    for (vit_kernel_stat& a : agg)
      if (std::strcmp(a.name, r.name) == 0) k = &a;
    if (!k) {
      vit_kernel_stat z{};
      std::snprintf(z.name, sizeof(z.name), "%s", r.name);
      z.mfma_bound = r.mfma ? 1 : 0;
      agg.push_back(z);
      k = &agg.back();
    }
    k->launches += 1;
    k->total_ms += ms;
    k->flops += r.flops;
    k->bytes += r.bytes;
  }
  for (size_t i = 0; i < agg.size() && (int32_t)i < max_stats; ++i) stats[i] = agg[i];
  if (n_stats) *n_stats = (int32_t)agg.size();
  return VIT_OK;
}

vit_status vit_debug_stage(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8,
                           void* ws, size_t ws_bytes, int32_t layer, int32_t step, void* dst,
                           size_t dst_bytes, void* stream) {
  VIT_TRY(check_common(ctx, plan, ws, ws_bytes));
  if (plan->n_rows == 0) return VIT_OK;
  if (!pixels_u8 || !dst) {
    set_error("pixels and dst must not be NULL");
    return VIT_E_ARG;
  }
  const int L = ctx->cfg.layers;
  const bool ok = (layer == -1 && (step == 0 || step == 1)) ||
                  (layer >= 0 && layer < L && step >= 1 && step <= 9) ||
                  (layer == L && step >= 1 && step <= 3);
  if (!ok) {
    set_error("no debug stage (%d, %d)", layer, step);
    return VIT_E_ARG;
  }
  Stop s;
  s.layer = layer;
  s.step = step;
  s.dst = dst;
  s.dst_bytes = dst_bytes;
  char* w = static_cast<char*>(ws);
  float* out = reinterpret_cast<float*>(w + plan->off_out);
  if (layer == L && step == 3) {
    // the final output goes straight to dst
    if (dst_bytes < (size_t)plan->n_units * ctx->cfg.out_dim * 4) {
      set_error("debug stage needs %zu bytes", (size_t)plan->n_units * ctx->cfg.out_dim * 4);
      return VIT_E_WORKSPACE;
    }
    s.layer = -2;
    return forward(ctx, plan, pixels_u8, nullptr, w, static_cast<float*>(dst),
                   static_cast<hipStream_t>(stream), true, s);
  }
  return forward(ctx, plan, pixels_u8, nullptr, w, out, static_cast<hipStream_t>(stream), true, s);
}

namespace {

vit_status capture_graph(const vit_ctx* ctx, const vit_plan* plan, void* ws, size_t ws_bytes,
                         void* stream, bool bucket, vit_graph** out) {
  if (!out) {
    set_error("out must not be NULL");
    return VIT_E_ARG;
  }
  *out = nullptr;
  VIT_TRY(check_common(ctx, plan, ws, ws_bytes));
  if (plan->n_rows == 0) {
    set_error("cannot capture an empty batch");
    return VIT_E_SHAPE;
  }
  hipStream_t user = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  // metadata is fixed for the plan: upload it once, outside the graph
  HIP_TRY(hipMemcpyAsync(w, plan->meta.data(), plan->meta.size(), hipMemcpyHostToDevice, user));
  HIP_TRY(hipStreamSynchronize(user));
  hipStream_t cap;
  HIP_TRY(hipStreamCreateWithFlags(&cap, hipStreamNonBlocking));
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cap);
    set_error("hipStreamBeginCapture: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  vit_status s = forward(ctx, plan, reinterpret_cast<const uint8_t*>(w + plan->off_pix), nullptr, w,
                         reinterpret_cast<float*>(w + plan->off_out), cap, false, Stop{}, nullptr, bucket);
  e = hipStreamEndCapture(cap, &graph);
  (void)hipStreamDestroy(cap);
  if (s != VIT_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return s;
  }
  if (e != hipSuccess) {
    set_error("hipStreamEndCapture: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    set_error("hipGraphInstantiate: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  vit_graph* g = new (std::nothrow) vit_graph();
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    set_error("out of host memory");
    return VIT_E_ARG;
  }
  g->ctx = ctx;
  g->plan = plan;
  g->ws = ws;
  g->graph = graph;
  g->exec = exec;
  g->bucket = bucket;
  if (bucket) {
    // pinned staging copy of the metadata region: the capacity plan's tables (cos/sin stay
    // valid for every smaller plan) with the per-batch parts rewritten at each launch
    hipEvent_t ev = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&g->staging), plan->meta.size(), hipHostMallocDefault) !=
            hipSuccess ||
        hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
      vit_graph_destroy(g);
      set_error("staging buffer for the bucketed graph: %s", hipGetErrorString(hipGetLastError()));
      return VIT_E_HIP;
    }
    g->staged = ev;
    std::memcpy(g->staging, plan->meta.data(), plan->meta.size());
  }
  *out = g;
  return VIT_OK;
}

}  // namespace

vit_status vit_graph_capture(const vit_ctx* ctx, const vit_plan* plan, void* ws, size_t ws_bytes,
                             void* stream, vit_graph** out) {
  return capture_graph(ctx, plan, ws, ws_bytes, stream, false, out);
}

vit_status vit_graph_capture_bucket(const vit_ctx* ctx, const vit_plan* plan, void* ws,
                                    size_t ws_bytes, void* stream, vit_graph** out) {
  return capture_graph(ctx, plan, ws, ws_bytes, stream, true, out);
}

vit_status vit_graph_launch_plan(vit_graph* g, const vit_plan* plan, void* stream) {
  if (!g || !plan) {
    set_error("graph and plan must not be NULL");
    return VIT_E_ARG;
  }
  if (!g->bucket) {
    set_error("graph was not captured with vit_graph_capture_bucket");
    return VIT_E_STATE;
  }
  const vit_plan* cap = g->plan;
  const vit_config& a = plan->cfg;
  const vit_config& b = cap->cfg;
  if (a.hidden != b.hidden || a.heads != b.heads || a.layers != b.layers || a.mlp_dim != b.mlp_dim ||
      a.window_px != b.window_px || a.out_dim != b.out_dim || plan->head_dim != cap->head_dim ||
      plan->split != cap->split || plan->f8 != cap->f8) {
    set_error("plan was built for another tower configuration than the captured one");
    return VIT_E_ARG;
  }
  if (plan->n_rows == 0) return VIT_OK;
  struct Fit {
    const char* what;
    int64_t need, have;
  } fits[] = {{"patches", plan->n_rows, cap->n_rows},
              {"pixel bytes", (int64_t)plan->pixel_bytes, (int64_t)cap->pixel_bytes},
              {"largest grid side", plan->max_pos, cap->max_pos},
              {"long attention units", plan->full.n_long, cap->full.n_long},
              {"short attention units", plan->full.n_short, cap->full.n_short},
              {"long window units", plan->win.n_long, cap->win.n_long},
              {"short window units", plan->win.n_short, cap->win.n_short}};
  for (const Fit& f : fits)
    if (f.need > f.have) {
      set_error("plan exceeds the bucket: %lld %s, capacity %lld", (long long)f.need, f.what,
                (long long)f.have);
      return VIT_E_SHAPE;
    }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the staging buffer is rewritten only once the previous upload from it has completed
  HIP_TRY(hipEventSynchronize(static_cast<hipEvent_t>(g->staged)));
  uint8_t* dst = g->staging;
  const uint8_t* src = plan->meta.data();
  auto put = [&](int64_t to, int64_t from, size_t bytes) {
    if (bytes) std::memcpy(dst + to, src + from, bytes);
  };
  put(cap->off_dims, plan->off_dims, sizeof(RunDims));
  put(cap->off_units, plan->off_units, (size_t)plan->n_units * sizeof(UnitDesc));
  put(cap->off_rowpos, plan->off_rowpos, (size_t)plan->n_rows * sizeof(int32_t));
  put(cap->off_unitdst, plan->off_unitdst, (size_t)plan->n_units * sizeof(int32_t));
  put(cap->full.off_long, plan->full.off_long, (size_t)plan->full.n_long * sizeof(AttnWork));
  put(cap->full.off_short, plan->full.off_short, (size_t)plan->full.n_short * sizeof(AttnWork));
  put(cap->win.off_long, plan->win.off_long, (size_t)plan->win.n_long * sizeof(AttnWork));
  put(cap->win.off_short, plan->win.off_short, (size_t)plan->win.n_short * sizeof(AttnWork));
  HIP_TRY(hipMemcpyAsync(g->ws, dst, cap->meta.size(), hipMemcpyHostToDevice, st));
  HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(g->staged), st));
  HIP_TRY(hipGraphLaunch(static_cast<hipGraphExec_t>(g->exec), st));
  return VIT_OK;
}

vit_status vit_graph_io(const vit_graph* g, uint8_t** pixels_in, float** out) {
  if (!g) {
    set_error("graph must not be NULL");
    return VIT_E_ARG;
  }
  char* w = static_cast<char*>(g->ws);
  if (pixels_in) *pixels_in = reinterpret_cast<uint8_t*>(w + g->plan->off_pix);
  if (out) *out = reinterpret_cast<float*>(w + g->plan->off_out);
  return VIT_OK;
}

vit_status vit_graph_launch(vit_graph* g, void* stream) {
  if (!g) {
    set_error("graph must not be NULL");
    return VIT_E_ARG;
  }
  HIP_TRY(hipGraphLaunch(static_cast<hipGraphExec_t>(g->exec), static_cast<hipStream_t>(stream)));
  return VIT_OK;
}

void vit_graph_destroy(vit_graph* g) {
  if (!g) return;
  if (g->staged) {
    (void)hipEventSynchronize(static_cast<hipEvent_t>(g->staged));
    (void)hipEventDestroy(static_cast<hipEvent_t>(g->staged));
  }
  if (g->staging) (void)hipHostFree(g->staging);
  if (g->exec) (void)hipGraphExecDestroy(static_cast<hipGraphExec_t>(g->exec));
  if (g->graph) (void)hipGraphDestroy(static_cast<hipGraph_t>(g->graph));
  delete g;
}

void vit_destroy(vit_ctx* ctx) {
  if (!ctx) return;
  if (ctx->w.arena) (void)hipFree(ctx->w.arena);
  delete ctx;
}

}  // extern "C"
