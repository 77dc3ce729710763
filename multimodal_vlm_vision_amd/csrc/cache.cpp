// Host side of the serving helpers around the path: the vision-embedding cache and the device
// resize entry point (resize.hip).
//
// Vision-embedding cache: merged embeddings reused across calls, keyed by the content of an
// item's uint8 pixels and its grid ("vLLM multimodal inference | ViT performance
// optimisation", section 2.3 lists a vision-embedding cache shared across requests).
//
// Keys come from the pixel hash kernel (pixel_hash.hip).  Entries live in a caller-owned
// device arena used as a ring: an entry is written at the ring head (wrapping to the start
// when it does not fit before the end) after evicting every older entry it overlaps, so
// eviction is first-in first-out.  vit_encode_cached computes the batch's keys (one
// device-to-host copy and a stream synchronisation: the split into hits and misses is a host
// decision), gathers the misses' pixels into the workspace's pixel region of a plan built for
// the misses alone, encodes that plan, then assembles the output in item order from the
// arena (hits) and the misses' output, and inserts the misses.  All copies are asynchronous
// on the caller's stream.  Not thread-safe: one cache per thread or external locking.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "vit_internal.h"

namespace {

struct Key {
  uint64_t h0, h1;
  int32_t t, h, w, nf;
  bool operator==(const Key& o) const {
    return h0 == o.h0 && h1 == o.h1 && t == o.t && h == o.h && w == o.w && nf == o.nf;
  }
};
struct KeyHash {
  size_t operator()(const Key& k) const { return (size_t)(k.h0 ^ (k.h1 * 0x9e3779b97f4a7c15ull)); }
};
struct Entry {
  size_t off = 0, bytes = 0;
};

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

#define VIT_TRY(expr)          \
  do {                         \
    vit_status s_ = (expr);    \
    if (s_ != VIT_OK) return s_; \
  } while (0)

#define HIP_OK(x)                                                       \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      vitmi::set_error("%s: %s", #x, hipGetErrorString(e_));            \
      return VIT_E_HIP;                                                 \
    }                                                                   \
  } while (0)

struct ItemInfo {
  int64_t px_off = 0, px_bytes = 0, unit_off = 0, units = 0;
};

std::vector<ItemInfo> item_layout(const vit_plan* p) {
  std::vector<ItemInfo> v((size_t)p->n_items);
  int64_t px = 0, u = 0;
  for (int i = 0; i < p->n_items; ++i) {
    const int64_t t = p->grid[3 * i], h = p->grid[3 * i + 1], w = p->grid[3 * i + 2];
    const int64_t nf = p->nframes[i];
    v[i].px_off = px;
    v[i].px_bytes = nf * (14 * h) * (14 * w) * 3;
    v[i].unit_off = u;
    v[i].units = t * h * w / 4;
    px += v[i].px_bytes;
    u += v[i].units;
  }
  return v;
}

}  // namespace

struct vit_cache {
  const vit_ctx* ctx = nullptr;
  char* arena = nullptr;
  size_t cap = 0, head = 0, used = 0;
  std::deque<Key> fifo;   // insertion order
  std::unordered_map<Key, Entry, KeyHash> map;
};

namespace {

// The batch's keys (n_items x {h0, h1}, final mix applied).  Uses the start of ws (the
// metadata region, which every encode rewrites) for the item table and the partial sums.
vit_status batch_keys(const vit_plan* plan, const uint8_t* pixels, char* ws, hipStream_t st,
                      std::vector<uint64_t>& keys) {
  const int n = plan->n_items;
  keys.assign(2 * (size_t)n, 0);
  if (n == 0) return VIT_OK;
  if (reinterpret_cast<uintptr_t>(pixels) % 16) {
    vitmi::set_error("pixels must be 16-byte aligned for the pixel hash");
    return VIT_E_ARG;
  }
  const std::vector<ItemInfo> L = item_layout(plan);
  std::vector<int64_t> table(2 * (size_t)n);
  int64_t max_words = 0;
  for (int i = 0; i < n; ++i) {
    table[2 * i] = L[i].px_off;
    table[2 * i + 1] = L[i].px_bytes / 8;
    max_words = std::max(max_words, L[i].px_bytes / 8);
  }
  const size_t tbytes = vitmi::round_up(16 * (int64_t)n, 256);
  if ((size_t)plan->off_x < tbytes + 16 * (size_t)n) {
    vitmi::set_error("workspace metadata region too small for the pixel keys");
    return VIT_E_WORKSPACE;
  }
  int64_t* items_dev = reinterpret_cast<int64_t*>(ws);
  uint64_t* sums_dev = reinterpret_cast<uint64_t*>(ws + tbytes);
  HIP_OK(hipMemcpyAsync(items_dev, table.data(), 16 * (size_t)n, hipMemcpyHostToDevice, st));
  VIT_TRY(vitmi::launch_pixel_hash(pixels, items_dev, n, max_words, sums_dev, st));
  HIP_OK(hipMemcpyAsync(keys.data(), sums_dev, 16 * (size_t)n, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  const uint64_t G[2] = {0x9e3779b97f4a7c15ull, 0xd1b54a32d192ed03ull};
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < 2; ++j) keys[2 * i + j] = mix64(keys[2 * i + j] ^ ((uint64_t)L[i].px_bytes * G[j]));
  return VIT_OK;
}

void evict_overlapping(vit_cache* c, size_t off, size_t bytes) {
  while (!c->fifo.empty()) {
    // entries are written in ring order, so the oldest ones are the ones the head reaches
    bool any = false;
    for (auto it = c->fifo.begin(); it != c->fifo.end();) {
      const Entry& e = c->map[*it];
      if (e.off < off + bytes && off < e.off + e.bytes) {
        c->used -= e.bytes;
        c->map.erase(*it);
        it = c->fifo.erase(it);
        any = true;
      } else {
        ++it;
      }
    }
    if (!any) break;
  }
}

}  // namespace

extern "C" {

vit_status vit_cache_create(const vit_ctx* ctx, void* arena, size_t arena_bytes, vit_cache** out) {
  if (!ctx || !out || (!arena && arena_bytes)) {
    vitmi::set_error("ctx and out must not be NULL (and arena unless arena_bytes is 0)");
    return VIT_E_ARG;
  }
  if (reinterpret_cast<uintptr_t>(arena) % 256) {
    vitmi::set_error("arena must be 256-byte aligned");
    return VIT_E_ARG;
  }
  vit_cache* c = new (std::nothrow) vit_cache();
  if (!c) {
    vitmi::set_error("out of host memory");
    return VIT_E_ARG;
  }
  c->ctx = ctx;
  c->arena = static_cast<char*>(arena);
  c->cap = arena_bytes;
  *out = c;
  return VIT_OK;
}

void vit_cache_destroy(vit_cache* c) { delete c; }

vit_status vit_cache_stats(const vit_cache* c, int64_t* entries, size_t* bytes_used) {
  if (!c) {
    vitmi::set_error("cache must not be NULL");
    return VIT_E_ARG;
  }
  if (entries) *entries = (int64_t)c->map.size();
  if (bytes_used) *bytes_used = c->used;
  return VIT_OK;
}

vit_status vit_pixel_keys(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8, void* ws,
                          size_t ws_bytes, uint64_t* keys, void* stream) {
  VIT_TRY(vitmi::check_plan_ws(ctx, plan, ws, ws_bytes));
  if (plan->n_items == 0) return VIT_OK;
  if (!pixels_u8 || !keys) {
    vitmi::set_error("pixels and keys must not be NULL");
    return VIT_E_ARG;
  }
  std::vector<uint64_t> k;
  VIT_TRY(batch_keys(plan, pixels_u8, static_cast<char*>(ws), static_cast<hipStream_t>(stream), k));
  std::memcpy(keys, k.data(), k.size() * sizeof(uint64_t));
  return VIT_OK;
}

vit_status vit_encode_cached(const vit_ctx* ctx, vit_cache* cache, const vit_plan* plan,
                             const uint8_t* pixels_u8, void* ws, size_t ws_bytes, float* out, void* stream,
                             int32_t* n_hits) {
  if (n_hits) *n_hits = 0;
  if (!cache) {
    vitmi::set_error("cache must not be NULL");
    return VIT_E_ARG;
  }
  VIT_TRY(vitmi::check_plan_ws(ctx, plan, ws, ws_bytes));
  if (cache->ctx != ctx) {
    vitmi::set_error("the cache belongs to another context");
    return VIT_E_ARG;
  }
  if (plan->n_rows == 0) return VIT_OK;
  if (!pixels_u8 || !out) {
    vitmi::set_error("pixels and out must not be NULL");
    return VIT_E_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  std::vector<uint64_t> keys;
  VIT_TRY(batch_keys(plan, pixels_u8, w, st, keys));
  const std::vector<ItemInfo> L = item_layout(plan);
  const size_t row_bytes = (size_t)ctx->cfg.out_dim * sizeof(float);
  const int n = plan->n_items;

  std::vector<Key> K((size_t)n);
  std::vector<int> miss;
  std::vector<int32_t> mgrid, mframes;
  for (int i = 0; i < n; ++i) {
    K[i] = Key{keys[2 * i], keys[2 * i + 1], plan->grid[3 * i], plan->grid[3 * i + 1], plan->grid[3 * i + 2],
               plan->nframes[i]};
    if (!cache->map.count(K[i])) {
      // a repeated item inside this batch is encoded once per occurrence
      miss.push_back(i);
      mgrid.insert(mgrid.end(), &plan->grid[3 * i], &plan->grid[3 * i] + 3);
      mframes.push_back(plan->nframes[i]);
    }
  }
  // hits: straight from the arena
  for (int i = 0; i < n; ++i) {
    auto it = cache->map.find(K[i]);
    if (it == cache->map.end()) continue;
    HIP_OK(hipMemcpyAsync(reinterpret_cast<char*>(out) + (size_t)L[i].unit_off * row_bytes,
                          cache->arena + it->second.off, it->second.bytes, hipMemcpyDeviceToDevice, st));
  }
  if (n_hits) *n_hits = n - (int32_t)miss.size();
  if (miss.empty()) return VIT_OK;

  // misses: one plan for them alone, pixels gathered into that plan's pixel region of ws.  That
  // plan runs no key-split attention units, so a cached item's rows do not depend on which
  // other items missed with it, and every workspace region of the plan is at most the batch's.
  vit_plan* sub = nullptr;
  VIT_TRY(vitmi::create_plan(ctx, mgrid.data(), mframes.data(), (int32_t)miss.size(), false, &sub));
  struct PlanGuard {
    vit_plan* p;
    ~PlanGuard() { vit_plan_destroy(p); }
  } guard{sub};
  if (sub->ws_bytes > ws_bytes) {   // cannot happen: every region grows with the batch
    vitmi::set_error("workspace too small for the uncached items");
    return VIT_E_WORKSPACE;
  }
  size_t px = 0;
  for (int i : miss) {
    HIP_OK(hipMemcpyAsync(w + sub->off_pix + px, pixels_u8 + L[i].px_off, (size_t)L[i].px_bytes,
                          hipMemcpyDeviceToDevice, st));
    px += (size_t)L[i].px_bytes;
  }
  float* mout = reinterpret_cast<float*>(w + sub->off_out);
  VIT_TRY(vit_encode(ctx, sub, reinterpret_cast<const uint8_t*>(w + sub->off_pix), ws, ws_bytes, mout, stream));
  // scatter the misses' rows into the batch output and insert them
  size_t mrow = 0;
  for (int i : miss) {
    const size_t bytes = (size_t)L[i].units * row_bytes;
    const char* src = reinterpret_cast<const char*>(mout) + mrow * row_bytes;
    HIP_OK(hipMemcpyAsync(reinterpret_cast<char*>(out) + (size_t)L[i].unit_off * row_bytes, src, bytes,
                          hipMemcpyDeviceToDevice, st));
    mrow += (size_t)L[i].units;
    if (bytes == 0 || bytes > cache->cap || cache->map.count(K[i])) continue;
    size_t off = cache->head;
    if (off + bytes > cache->cap) off = 0;
    evict_overlapping(cache, off, bytes);
    HIP_OK(hipMemcpyAsync(cache->arena + off, src, bytes, hipMemcpyDeviceToDevice, st));
    cache->map[K[i]] = Entry{off, bytes};
    cache->fifo.push_back(K[i]);
    cache->used += bytes;
    cache->head = vitmi::round_up((int64_t)(off + bytes), 256);
  }
  return VIT_OK;
}

int32_t vit_resize_side(int32_t pixels) { return pixels < 1 ? 0 : vitmi::resize_side(pixels); }

vit_status vit_resize_u8(const uint8_t* src, int32_t sh, int32_t sw, int32_t frames, uint8_t* dst,
                         size_t dst_bytes, void* stream) {
  if (!src || !dst || sh < 1 || sw < 1 || frames < 1) {
    vitmi::set_error("resize: src/dst must not be NULL and sh, sw, frames >= 1 (got %d, %d, %d)", sh, sw, frames);
    return VIT_E_ARG;
  }
  if (sh > 8192 || sw > 8192) {
    vitmi::set_error("resize: sides must be <= 8192 pixels");
    return VIT_E_SHAPE;
  }
  const int dh = vitmi::resize_side(sh), dw = vitmi::resize_side(sw);
  const size_t need = (size_t)frames * dh * dw * 3, have = (size_t)frames * sh * sw * 3;
  if (dst_bytes < need) {
    vitmi::set_error("resize: dst needs %zu bytes, got %zu", need, dst_bytes);
    return VIT_E_WORKSPACE;
  }
  if (need / 256 >= ((size_t)1 << 31)) {
    vitmi::set_error("resize: output too large");
    return VIT_E_SHAPE;
  }
  if (reinterpret_cast<uintptr_t>(src) % 4 || reinterpret_cast<uintptr_t>(dst) % 4) {
    vitmi::set_error("resize: src and dst must be 4-byte aligned");
    return VIT_E_ARG;
  }
  const uint8_t* s0 = src;
  const uint8_t* d0 = dst;
  if (s0 < d0 + need && d0 < s0 + have) {
    vitmi::set_error("resize: src and dst must not overlap");
    return VIT_E_ARG;
  }
  return vitmi::launch_resize(src, sh, sw, frames, dst, dh, dw, stream);
}

}  // extern "C"
