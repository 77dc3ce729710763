// Weight intake and packing.
//
// Separate q/k/v projections are stacked into one qkv matrix (vLLM PR #55370
// report, key code: the vision checkpoints' q/k/v are mapped onto a fused
// qkv).  Packing then lays the weights out for the GEMM epilogues:
//  - qkv: the q and k rows are reordered so that the two members of every
//    rotary pair (k, k + head_dim/2) land 32 columns apart inside one
//    64-column block; the RoPE epilogue then finds both in one lane;
//  - SwiGLU gate/up: interleaved per 32 rows so that gate j and up j share a lane;
//  - the patch-embed K (1176) and the MLP width are zero-padded to multiples of 64.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>

#include "vit_internal.h"

namespace vitmi {

uint16_t f32_to_bf16_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP 8-bit floating point E4M3 (OFP8 specification, 2023): sign, 4 exponent bits with bias
// 7, 3 mantissa bits, no infinities, S.1111.111 the only NaN, largest finite value 448.
// Round to nearest even; magnitudes at or above 448 saturate to 448.
uint8_t f32_to_e4m3_bits(float f) {
  const uint8_t sign = std::signbit(f) ? 0x80 : 0;
  const double a = std::fabs((double)f);
  if (std::isnan(f)) return 0x7f;
  if (a >= 448.0) return sign | 0x7e;
  int e2;
  (void)std::frexp(a, &e2);                  // a in [2^(e2-1), 2^e2)
  const int E = a == 0.0 ? -6 : std::max(e2 - 1, -6);   // below 2^-6: subnormal quantum 2^-9
  const double q = std::ldexp(1.0, E - 3);
  const double r = std::nearbyint(a / q) * q;   // the default rounding mode is to nearest even
  if (r >= 448.0) return sign | 0x7e;
  if (r < std::ldexp(1.0, -6)) return sign | (uint8_t)(r / std::ldexp(1.0, -9));   // subnormal (or 0)
  int er;
  (void)std::frexp(r, &er);
  const int Er = er - 1;                     // r may have rounded up into the next binade
  const int mant = (int)(r / std::ldexp(1.0, Er - 3)) - 8;
  return sign | (uint8_t)((Er + 7) << 3) | (uint8_t)mant;
}

// IEEE 754 binary16: sign, 5 exponent bits with bias 15, 10 fraction bits; subnormals on a
// 2^-24 grid below 2^-14; largest finite value 65504.  Round to nearest even; magnitudes that
// round past 65504 become infinity.
uint16_t f32_to_f16_bits(float f) {
  const uint16_t sign = std::signbit(f) ? 0x8000 : 0;
  if (std::isnan(f)) return 0x7e00;
  const double a = std::fabs((double)f);
  if (std::isinf(f)) return sign | 0x7c00;
  if (a < std::ldexp(1.0, -14)) {                           // subnormal range (or 0)
    const double k = std::nearbyint(a / std::ldexp(1.0, -24));   // default mode: to nearest even
    return sign | (uint16_t)k;   // k == 1024 encodes the smallest normal number, 2^-14
  }
  int e2;
  (void)std::frexp(a, &e2);      // a in [2^(e2-1), 2^e2)
  int E = e2 - 1;
  double k = std::nearbyint((a / std::ldexp(1.0, E) - 1.0) * 1024.0);
  if (k == 1024.0) {             // rounded up into the next binade
    k = 0.0;
    E += 1;
  }
  if (E > 15) return sign | 0x7c00;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)k;
}

static float bf16_bits_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

vit_status store_weight(vit_ctx* ctx, const char* name, int32_t dtype, const int64_t* shape,
                        int32_t ndim, const void* host_ptr) {
  if (!name || !host_ptr || (ndim > 0 && !shape) || ndim < 1 || ndim > 8) {
    set_error("vit_load_weight: bad argument");
    return VIT_E_ARG;
  }
  if (ctx->finalized) {
    set_error("vit_load_weight after vit_finalize_weights");
    return VIT_E_STATE;
  }
  if (dtype != VIT_F32 && dtype != VIT_BF16) {
    set_error("vit_load_weight %s: dtype must be VIT_F32 or VIT_BF16", name);
    return VIT_E_ARG;
  }
  if (ctx->host.count(name)) {
    set_error("vit_load_weight: duplicate weight %s", name);
    return VIT_E_WEIGHTS;
  }
  HostTensor t;
  int64_t n = 1;
  for (int i = 0; i < ndim; ++i) {
    if (shape[i] <= 0) {
      set_error("vit_load_weight %s: non-positive dimension", name);
      return VIT_E_SHAPE;
    }
    t.shape.push_back(shape[i]);
    n *= shape[i];
  }
  t.data.resize(n);
  if (dtype == VIT_F32) {
    std::memcpy(t.data.data(), host_ptr, n * 4);
  } else {
    const uint16_t* s = static_cast<const uint16_t*>(host_ptr);
    for (int64_t i = 0; i < n; ++i) t.data[i] = bf16_bits_to_f32(s[i]);
  }
  ctx->host.emplace(name, std::move(t));
  return VIT_OK;
}

namespace {

struct Packer {
  vit_ctx* ctx;
  std::vector<uint8_t> blob;   // host image of the device arena
  std::string err;

  const HostTensor* get(const std::string& name, std::initializer_list<int64_t> shape) {
    auto it = ctx->host.find(name);
    if (it == ctx->host.end()) {
      err = "missing weight " + name;
      return nullptr;
    }
    const HostTensor& t = it->second;
    int64_t want = 1, have = 1;
    for (int64_t s : shape) want *= s;
    for (int64_t s : t.shape) have *= s;
    bool ok = want == have && !t.shape.empty() && t.shape[0] == *shape.begin();
    if (!ok) {
      err = "weight " + name + " has the wrong shape";
      return nullptr;
    }
    return &t;
  }
  size_t reserve(size_t bytes) {
    size_t off = round_up((int64_t)blob.size(), 256);
    blob.resize(off + bytes);
    return off;
  }
  // rows x cols bf16 GEMM operand in the blocked layout (kt_index); element (r, c) = src(r, c)
  // via a callback.  Every packed matrix has rows a multiple of 64 and cols of 32 (checked by
  // the configuration and the padding of the K dimensions).
  template <class F>
  size_t mat(int64_t rows, int64_t cols, F src) {
    size_t off = reserve((size_t)rows * cols * 2);
    uint16_t* d = reinterpret_cast<uint16_t*>(blob.data() + off);
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; ++c) d[kt_index(r, c, cols)] = f32_to_bf16_bits(src(r, c));
    return off;
  }
  // e4m3 copy of the same matrix for the compensated products (kt8_index layout; rows a
  // multiple of 64): the bf16-rounded value of row r times 2^e_r, e_r the largest power that
  // keeps the row's largest magnitude within 448; scale_off receives the rows' E8M0 bytes
  // 127 - e_r (so the GEMM's scaled MFMA multiplies row r back by 2^-e_r).
  template <class F>
  size_t mat8(int64_t rows, int64_t cols, F src, size_t& scale_off) {
    std::vector<float> row(cols);
    std::vector<uint8_t> sc(rows);
    size_t off = reserve((size_t)rows * cols);
    for (int64_t r = 0; r < rows; ++r) {
      double mx = 0;
      for (int64_t c = 0; c < cols; ++c) {
        row[c] = bf16_bits_to_f32(f32_to_bf16_bits(src(r, c)));
        mx = std::max(mx, (double)std::fabs(row[c]));
      }
      int e = 0;
      if (mx > 0) {
        int e2;
        const double m = std::frexp(mx, &e2);   // mx = m 2^e2, m in [0.5, 1)
        e = (m * 512.0 <= 448.0 ? 9 : 8) - e2;
        e = std::min(std::max(e, -127), 127);
      }
      sc[r] = (uint8_t)(127 - e);
      uint8_t* d = blob.data() + off;
      for (int64_t c = 0; c < cols; ++c) d[kt8_index(r, c, cols)] = f32_to_e4m3_bits(std::ldexp(row[c], e));
    }
    scale_off = reserve((size_t)rows);
    std::memcpy(blob.data() + scale_off, sc.data(), rows);
    return off;
  }
  // float16 copy for the float16 activation form: the bf16-rounded value of (r, c) times 2^e,
  // one e for the whole matrix, the largest power that keeps its largest magnitude below 2^15.
  // The conversion is exact for every value above 2^-39 of that magnitude (smaller ones land
  // on float16's subnormal grid, an error below 2^-40 of the largest weight).  acc_scale
  // receives 2^-e, which the GEMM epilogue multiplies the accumulators by (exact).
  template <class F>
  size_t mat16(int64_t rows, int64_t cols, F src, float& acc_scale) {
    double mx = 0;
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; ++c)
        mx = std::max(mx, (double)std::fabs(bf16_bits_to_f32(f32_to_bf16_bits(src(r, c)))));
    int e = 0;
    if (mx > 0) {
      int e2;
      (void)std::frexp(mx, &e2);   // mx < 2^e2
      e = std::min(std::max(15 - e2, -100), 100);
    }
    acc_scale = (float)std::ldexp(1.0, -e);
    size_t off = reserve((size_t)rows * cols * 2);
    uint16_t* d = reinterpret_cast<uint16_t*>(blob.data() + off);
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; ++c) {
        const float w = bf16_bits_to_f32(f32_to_bf16_bits(src(r, c)));
        d[kt_index(r, c, cols)] = f32_to_f16_bits((float)std::ldexp((double)w, e));
      }
    return off;
  }
  template <class F>
  size_t vec(int64_t n, F src) {
    size_t off = reserve((size_t)n * 4);
    float* d = reinterpret_cast<float*>(blob.data() + off);
    for (int64_t i = 0; i < n; ++i) d[i] = src(i);
    return off;
  }
};

}  // namespace

vit_status finalize_weights(vit_ctx* ctx, void* stream) {
  if (ctx->finalized) {
    set_error("vit_finalize_weights called twice");
    return VIT_E_STATE;
  }
  const vit_config& c = ctx->cfg;
  const int64_t d = c.hidden, hd = ctx->head_dim, mlp = c.mlp_dim, mp = ctx->mlp_pad;
  const int64_t md = 4 * d, od = c.out_dim;
  const int64_t r = hd / 2;   // rotary pairs per head
  Packer P{ctx, {}, {}};

  struct LayerOff {
    size_t n1g, n1b, n2g, n2b, qkv_w, qkv_b, proj_w, proj_b, fc1_w, fc1_b, fc2_w, fc2_b;
    size_t qkv_w8 = 0, qkv_s8 = 0, proj_w8 = 0, proj_s8 = 0, fc1_w8 = 0, fc1_s8 = 0, fc2_w8 = 0, fc2_s8 = 0;
    float qkv_sc = 1.0f, proj_sc = 1.0f, fc1_sc = 1.0f, fc2_sc = 1.0f;   // float16 weight scales
  };
  const bool f8 = ctx->f8;
  const bool f16 = ctx->f16;
  float m1sc = 1.0f, m2sc = 1.0f;   // merger float16 weight scales
  std::vector<LayerOff> lo(c.layers);

  size_t lut_off = P.reserve(3 * 256 * 2);
  std::memcpy(P.blob.data() + lut_off, ctx->lut, sizeof(ctx->lut));

  const HostTensor* pe = P.get("pe.w", {d, kFeat});
  if (!pe) goto fail;
  size_t pe_off;
  pe_off = P.mat(d, kFeatPad, [&](int64_t o, int64_t k) {
    return k < kFeat ? pe->data[o * kFeat + k] : 0.f;
  });

  for (int l = 0; l < c.layers; ++l) {
    const std::string p = "blk" + std::to_string(l) + ".";
    LayerOff& L = lo[l];
    auto norm = [&](const std::string& nm, size_t& go, size_t& bo) -> bool {
      const HostTensor* g = P.get(p + nm + ".g", {d});
      if (!g) return false;
      go = P.vec(d, [&](int64_t i) { return g->data[i]; });
      if (c.norm_kind == VIT_NORM_LAYER) {
        const HostTensor* b = P.get(p + nm + ".b", {d});
        if (!b) return false;
        bo = P.vec(d, [&](int64_t i) { return b->data[i]; });
      } else {
        bo = P.vec(d, [&](int64_t) { return 0.f; });
      }
      return true;
    };
    if (!norm("n1", L.n1g, L.n1b) || !norm("n2", L.n2g, L.n2b)) goto fail;

    // fused qkv: either given stacked or as q/k/v
    std::vector<float> wq, bq;
    if (ctx->host.count(p + "qkv.w")) {
      const HostTensor* w = P.get(p + "qkv.w", {3 * d, d});
      const HostTensor* b = P.get(p + "qkv.b", {3 * d});
      if (!w || !b) goto fail;
      wq = w->data;
      bq = b->data;
    } else {
      for (const char* s : {"q", "k", "v"}) {
        const HostTensor* w = P.get(p + s + ".w", {d, d});
        const HostTensor* b = P.get(p + s + ".b", {d});
        if (!w || !b) goto fail;
        wq.insert(wq.end(), w->data.begin(), w->data.end());
        bq.insert(bq.end(), b->data.begin(), b->data.end());
      }
    }
    // packed column j of the q (k) part: block j/64, slot s = j%64; pair = 32*(j/64) + s%32;
    // slot < 32 holds the pair's first member, slot >= 32 its partner (+ head_dim/2)
    auto src_row = [&](int64_t j) -> int64_t {
      const int64_t part = j / d, jj = j % d;
      if (part == 2) return j;
      const int64_t s = jj % 64, pair = 32 * (jj / 64) + s % 32;
      const int64_t head = pair / r, kk = pair % r;
      return part * d + head * hd + kk + (s < 32 ? 0 : r);
    };
    auto qkv_src = [&](int64_t j, int64_t k) { return wq[src_row(j) * d + k]; };
    L.qkv_w = f16 ? P.mat16(3 * d, d, qkv_src, L.qkv_sc) : P.mat(3 * d, d, qkv_src);
    if (f8) L.qkv_w8 = P.mat8(3 * d, d, qkv_src, L.qkv_s8);
    L.qkv_b = P.vec(3 * d, [&](int64_t j) { return bq[src_row(j)]; });

    const HostTensor* pw = P.get(p + "proj.w", {d, d});
    const HostTensor* pb = P.get(p + "proj.b", {d});
    if (!pw || !pb) goto fail;
    auto proj_src = [&](int64_t o, int64_t k) { return pw->data[o * d + k]; };
    L.proj_w = f16 ? P.mat16(d, d, proj_src, L.proj_sc) : P.mat(d, d, proj_src);
    if (f8) L.proj_w8 = P.mat8(d, d, proj_src, L.proj_s8);
    L.proj_b = P.vec(d, [&](int64_t i) { return pb->data[i]; });

    if (c.mlp_kind == VIT_MLP_GELU) {
      const HostTensor* w1 = P.get(p + "fc1.w", {mlp, d});
      const HostTensor* b1 = P.get(p + "fc1.b", {mlp});
      const HostTensor* w2 = P.get(p + "fc2.w", {d, mlp});
      const HostTensor* b2 = P.get(p + "fc2.b", {d});
      if (!w1 || !b1 || !w2 || !b2) goto fail;
      auto fc1_src = [&](int64_t o, int64_t k) { return o < mlp ? w1->data[o * d + k] : 0.f; };
      auto fc2_src = [&](int64_t o, int64_t k) { return k < mlp ? w2->data[o * mlp + k] : 0.f; };
      L.fc1_w = f16 ? P.mat16(mp, d, fc1_src, L.fc1_sc) : P.mat(mp, d, fc1_src);
      L.fc1_b = P.vec(mp, [&](int64_t o) { return o < mlp ? b1->data[o] : 0.f; });
      L.fc2_w = f16 ? P.mat16(d, mp, fc2_src, L.fc2_sc) : P.mat(d, mp, fc2_src);
      if (f8) {
        L.fc1_w8 = P.mat8(mp, d, fc1_src, L.fc1_s8);
        L.fc2_w8 = P.mat8(d, mp, fc2_src, L.fc2_s8);
      }
      L.fc2_b = P.vec(d, [&](int64_t i) { return b2->data[i]; });
    } else {
      const HostTensor* wg = P.get(p + "gate.w", {mlp, d});
      const HostTensor* bg = P.get(p + "gate.b", {mlp});
      const HostTensor* wu = P.get(p + "up.w", {mlp, d});
      const HostTensor* bu = P.get(p + "up.b", {mlp});
      const HostTensor* wd = P.get(p + "down.w", {d, mlp});
      const HostTensor* bd = P.get(p + "down.b", {d});
      if (!wg || !bg || !wu || !bu || !wd || !bd) goto fail;
      // packed row j: block j/64; slot < 32 -> gate row, slot >= 32 -> up row, index 32*(j/64) + slot%32
      auto gu = [&](int64_t j, bool& is_up) -> int64_t {
        const int64_t s = j % 64;
        is_up = s >= 32;
        return 32 * (j / 64) + s % 32;
      };
      auto fc1_src = [&](int64_t j, int64_t k) {
        bool up;
        const int64_t o = gu(j, up);
        if (o >= mlp) return 0.f;
        return (up ? wu : wg)->data[o * d + k];
      };
      auto fc2_src = [&](int64_t o, int64_t k) { return k < mlp ? wd->data[o * mlp + k] : 0.f; };
      L.fc1_w = f16 ? P.mat16(2 * mp, d, fc1_src, L.fc1_sc) : P.mat(2 * mp, d, fc1_src);
      L.fc1_b = P.vec(2 * mp, [&](int64_t j) {
        bool up;
        const int64_t o = gu(j, up);
        if (o >= mlp) return 0.f;
        return (up ? bu : bg)->data[o];
      });
      L.fc2_w = f16 ? P.mat16(d, mp, fc2_src, L.fc2_sc) : P.mat(d, mp, fc2_src);
      L.fc2_b = P.vec(d, [&](int64_t i) { return bd->data[i]; });
      if (f8) {
        L.fc1_w8 = P.mat8(2 * mp, d, fc1_src, L.fc1_s8);
        L.fc2_w8 = P.mat8(d, mp, fc2_src, L.fc2_s8);
      }
    }
  }

  size_t mqg, mqb, m1w, m1b, m2w, m2b, m1w8, m1s8, m2w8, m2s8;
  {
    const HostTensor* g = P.get("mrg.nq.g", {d});
    if (!g) goto fail;
    mqg = P.vec(d, [&](int64_t i) { return g->data[i]; });
    if (c.norm_kind == VIT_NORM_LAYER) {
      const HostTensor* b = P.get("mrg.nq.b", {d});
      if (!b) goto fail;
      mqb = P.vec(d, [&](int64_t i) { return b->data[i]; });
    } else {
      mqb = P.vec(d, [&](int64_t) { return 0.f; });
    }
    const HostTensor* w1 = P.get("mrg.fc1.w", {md, md});
    const HostTensor* b1 = P.get("mrg.fc1.b", {md});
    const HostTensor* w2 = P.get("mrg.fc2.w", {od, md});
    const HostTensor* b2 = P.get("mrg.fc2.b", {od});
    if (!w1 || !b1 || !w2 || !b2) goto fail;
    // merger input row = the merge unit's 4 patch rows concatenated (each stored as
    // [hi(d) | lo(d)] when split; the GEMM maps logical columns onto that layout)
    m1w8 = m1s8 = m2w8 = m2s8 = 0;
    auto m1_src = [&](int64_t o, int64_t k) { return w1->data[o * md + k]; };
    auto m2_src = [&](int64_t o, int64_t k) { return w2->data[o * md + k]; };
    m1w = f16 ? P.mat16(md, md, m1_src, m1sc) : P.mat(md, md, m1_src);
    m1b = P.vec(md, [&](int64_t i) { return b1->data[i]; });
    m2w = f16 ? P.mat16(od, md, m2_src, m2sc) : P.mat(od, md, m2_src);
    if (f8) {
      m1w8 = P.mat8(md, md, m1_src, m1s8);
      m2w8 = P.mat8(od, md, m2_src, m2s8);
    }
    m2b = P.vec(od, [&](int64_t i) { return b2->data[i]; });
  }

  {
    hipError_t e = hipGetDevice(&ctx->device);
    if (e != hipSuccess) {
      set_error("hipGetDevice: %s", hipGetErrorString(e));
      return VIT_E_HIP;
    }
    e = hipDeviceGetAttribute(&ctx->n_cu, hipDeviceAttributeMultiprocessorCount, ctx->device);
    if (e != hipSuccess) {
      set_error("hipDeviceGetAttribute(multiprocessor count): %s", hipGetErrorString(e));
      return VIT_E_HIP;
    }
    vit_status ps = prepare_gemm_kernels();
    if (ps != VIT_OK) return ps;
    void* arena = nullptr;
    e = hipMalloc(&arena, P.blob.size());
    if (e != hipSuccess) {
      set_error("hipMalloc(%zu) for weights: %s", P.blob.size(), hipGetErrorString(e));
      return VIT_E_HIP;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    e = hipMemcpyAsync(arena, P.blob.data(), P.blob.size(), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      (void)hipFree(arena);
      set_error("weight upload: %s", hipGetErrorString(e));
      return VIT_E_HIP;
    }
    char* base = static_cast<char*>(arena);
    auto bf = [&](size_t o) { return reinterpret_cast<const uint16_t*>(base + o); };
    auto fl = [&](size_t o) { return reinterpret_cast<const float*>(base + o); };
    auto b8 = [&](size_t o) { return f8 ? reinterpret_cast<const uint8_t*>(base + o) : nullptr; };
    DeviceWeights& W = ctx->w;
    W.arena = arena;
    W.bytes = P.blob.size();
    W.lut = bf(lut_off);
    W.pe_w = bf(pe_off);
    W.layers.resize(c.layers);
    for (int l = 0; l < c.layers; ++l) {
      const LayerOff& L = lo[l];
      LayerW& X = W.layers[l];
      X.n1g = fl(L.n1g); X.n1b = fl(L.n1b); X.n2g = fl(L.n2g); X.n2b = fl(L.n2b);
      X.qkv_w = bf(L.qkv_w); X.qkv_b = fl(L.qkv_b);
      X.proj_w = bf(L.proj_w); X.proj_b = fl(L.proj_b);
      X.fc1_w = bf(L.fc1_w); X.fc1_b = fl(L.fc1_b);
      X.fc2_w = bf(L.fc2_w); X.fc2_b = fl(L.fc2_b);
      X.qkv_w8 = b8(L.qkv_w8); X.qkv_s8 = b8(L.qkv_s8);
      X.proj_w8 = b8(L.proj_w8); X.proj_s8 = b8(L.proj_s8);
      X.qkv_sc = L.qkv_sc; X.proj_sc = L.proj_sc; X.fc1_sc = L.fc1_sc; X.fc2_sc = L.fc2_sc;
      X.fc1_w8 = b8(L.fc1_w8); X.fc1_s8 = b8(L.fc1_s8);
      X.fc2_w8 = b8(L.fc2_w8); X.fc2_s8 = b8(L.fc2_s8);
    }
    W.mq_g = fl(mqg); W.mq_b = fl(mqb);
    W.m1_w = bf(m1w); W.m1_b = fl(m1b);
    W.m2_w = bf(m2w); W.m2_b = fl(m2b);
    W.m1_w8 = b8(m1w8); W.m1_s8 = b8(m1s8);
    W.m2_w8 = b8(m2w8); W.m2_s8 = b8(m2s8);
    W.m1_sc = m1sc; W.m2_sc = m2sc;
  }
  ctx->host.clear();
  ctx->finalized = true;
  return VIT_OK;

fail:
  set_error("vit_finalize_weights: %s", P.err.c_str());
  return VIT_E_WEIGHTS;
}

}  // namespace vitmi
