// Internal declarations shared by the host planner, the weight packer, the
// launch sequence and the HIP kernels of the vision-tower library.
#pragma once

#include <cstddef>
#include <cstdint>
#include <map>
#include <string>
#include <vector>

#include "../../include/vit.h"

namespace vitmi {

// ---------------------------------------------------------------- errors

void set_error(const char* fmt, ...);

// ---------------------------------------------------------------- fixed shape facts

constexpr int kPatch = 14;
constexpr int kTemporal = 2;
constexpr int kMerge = 2;
constexpr int kFeat = 3 * kTemporal * kPatch * kPatch;   // 1176 features per patch row
constexpr int kFeatPad = 1184;                            // padded to the GEMM K stage (32)
constexpr int kUnitPx = kMerge * kPatch;                  // 28-pixel side of a merge unit

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// ---------------------------------------------------------------- GEMM operand layout

// Every bf16 matrix that feeds a GEMM (weights, normalised patches, norm outputs,
// attention output, MLP activations) is stored in 1 KB blocks of 16 rows x 32 columns:
// blocks ordered by row group, then by column block; inside a block row r takes 64 bytes,
// its four 16-byte chunks permuted by kt_chunk.  A 64-lane 16-byte load then moves one
// whole block (eight full 128-byte lines instead of sixteen half lines), and the block
// lands in LDS already in the bank-conflict-free order the MFMA fragment reads need: a
// fragment read takes one chunk of 32 consecutive 64-byte rows, and with the chunk
// rotated by bits 3-4 of the row it runs at the LDS's full rate on gfx950 (measured with
// the LDS bank-conflict counter: rotations by bits 2-3 or 3-4 are conflict-free, ones
// that involve bit 1 take twice the cycles).
// Rows are padded to a multiple of 16, columns must be a multiple of 32.
constexpr int kt_chunk(int64_t r, int q) { return q ^ (int)((r >> 3) & 3); }
constexpr int64_t kt_index(int64_t r, int64_t c, int64_t cols) {
  return ((((r >> 4) * (cols >> 5) + (c >> 5)) << 9) | ((r & 15) << 5) |
          ((int64_t)kt_chunk(r, (int)((c >> 3) & 3)) << 3) | (c & 7));
}

// fp8 (OCP E4M3) matrices -- the residuals x - bf16(x) of the compensated activations and the
// weights' e4m3 copies -- use 1 KB blocks of 32 rows x 32 one-byte columns, ordered like
// kt_index (32-row group, then column block); inside a block row r takes 32 bytes and its two
// 16-byte chunks swap places when bit 3 of r is set, so a fragment read (32 consecutive rows,
// one chunk each) touches distinct banks in every 16-lane group.  Rows are padded to 32.
constexpr int64_t kt8_index(int64_t r, int64_t c, int64_t cols) {
  return ((((r >> 5) * (cols >> 5) + (c >> 5)) << 10) | ((r & 31) << 5) |
          ((((c >> 4) ^ (r >> 3)) & 1) << 4) | (c & 15));
}
// The residuals are stored times 2^kLoShift: |x - bf16(x)| <= 2^-8 |x|, so they stay within
// e4m3's maximum (448) for |x| <= 224 (larger ones saturate), and where they fall into e4m3's
// subnormal range their absolute error is at most 2^-10 * 2^-kLoShift = 2^-19.
constexpr int kLoShift = 9;

// bfloat16 round-to-nearest-even of a float, as raw bits (host side).
uint16_t f32_to_bf16_bits(float f);
// OCP E4M3 round-to-nearest-even of a float, saturating at +-448, as raw bits (host side).
uint8_t f32_to_e4m3_bits(float f);
// IEEE binary16 round-to-nearest-even of a float, as raw bits (host side).
uint16_t f32_to_f16_bits(float f);

// ---------------------------------------------------------------- device-side records

// One merge unit = a 2x2 block of patches = a 28x28 pixel block in each of the
// two temporal frames.  Byte offsets into the caller's packed pixel buffer.
struct UnitDesc {
  int64_t px_off;   // first byte of (frame slot 0, top-left pixel, channel 0)
  int32_t pitch;    // bytes per pixel row (W * 3)
  int32_t fstride;  // bytes from frame slot 0 to slot 1 (0: image, frame reused)
};
static_assert(sizeof(UnitDesc) == 16, "UnitDesc layout");

// One attention work unit: a block of queries of one segment (all heads via grid.y).
// It runs its queries against key blocks [kb0, kb1) of the segment (32 keys per block).  With
// part >= 0 the unit covers only part of the segment's keys and leaves its unnormalised
// output, running offset and softmax denominator in partial slot `part`, for the merge
// kernel; with part == -1 it covers all keys and writes the output itself.
struct AttnWork {
  int32_t seg_start;  // first internal row of the segment
  int32_t seg_len;    // rows in the segment
  int32_t q0;         // first query (relative to seg_start) of this unit
  int32_t kb0, kb1;   // key blocks of the unit
  int32_t part;       // partial slot, or -1
  int32_t pad[2];
};
static_assert(sizeof(AttnWork) == 32, "AttnWork layout");

// One merge of the partial units of a query block: partial slots [part0, part0 + n_parts).
struct AttnMerge {
  int32_t seg_start, seg_len, q0;
  int32_t part0, n_parts;
  int32_t pad[3];
};
static_assert(sizeof(AttnMerge) == 32, "AttnMerge layout");
constexpr int kAttnMaxParts = 16;   // parts of one query block at most

// Work lists for one kind of attention layer (item segments or windows).  The plain long list
// has one unit per 256-query block; the split list (used when n_merge > 0, by the eager
// forward and whole-forward graphs; bucketed graphs use the plain list) has the key-split
// units the planner chose to balance the launch's tail, and n_merge merges over n_parts
// partial slots.
struct AttnLists {
  int64_t off_long = 0;   // byte offset in the metadata blob
  int32_t n_long = 0;     // units of 256 queries (4-wave workgroups)
  int64_t off_short = 0;
  int32_t n_short = 0;    // units of 64 queries (1-wave workgroups)
  int64_t off_long_split = 0;
  int32_t n_long_split = 0;
  int64_t off_merge = 0;
  int32_t n_merge = 0;
  int32_t n_parts = 0;
  double sq_long = 0.0;   // sum of segment_length^2 over segments in each list
  double sq_short = 0.0;
};

// Batch sizes for a bucketed graph: the kernels of a graph captured for a capacity plan read
// these from device memory (the first 32 bytes of the plan's metadata region) instead of
// their launch-time counts, so any batch that fits the capacity replays the same graph.
struct RunDims {
  int32_t n_rows;       // patches N
  int32_t n_units;      // merge units N / 4
  int32_t full_long, full_short;   // attention work-list lengths, item segments
  int32_t win_long, win_short;     // and windows
  int32_t pad[2];
};
static_assert(sizeof(RunDims) == 32, "RunDims layout");

// Per-channel affine form of the normalisation, y = fma(x, a_c, b_c) in float32 then
// bf16 round-to-nearest-even.  Used only when the host has verified that it reproduces
// the exactly rounded table for all 768 (channel, byte) pairs.
struct NormAffine {
  float a[3], b[3];
};

// ---------------------------------------------------------------- weights

struct HostTensor {
  std::vector<int64_t> shape;
  std::vector<float> data;   // float32 values (exact copies of bf16 input if given as bf16)
};

struct LayerW {
  const float *n1g = nullptr, *n1b = nullptr, *n2g = nullptr, *n2b = nullptr;
  const uint16_t* qkv_w = nullptr;  const float* qkv_b = nullptr;   // [3d][d], q/k in RoPE pair order
  const uint16_t* proj_w = nullptr; const float* proj_b = nullptr;  // [d][d]
  const uint16_t* fc1_w = nullptr;  const float* fc1_b = nullptr;   // GELU [mlp_pad][d]; SwiGLU [2*mlp_pad][d]
  const uint16_t* fc2_w = nullptr;  const float* fc2_b = nullptr;   // [d][mlp_pad]
  // VIT_ACT_BF16F8: e4m3 copies of the weights that multiply compensated activations
  // (kt8_index layout, same shapes) and their per-row E8M0 scales (row n holds W[n] * 2^(127 - s[n]))
  const uint8_t* qkv_w8 = nullptr;  const uint8_t* qkv_s8 = nullptr;
  const uint8_t* proj_w8 = nullptr; const uint8_t* proj_s8 = nullptr;
  const uint8_t* fc1_w8 = nullptr;  const uint8_t* fc1_s8 = nullptr;
  const uint8_t* fc2_w8 = nullptr;  const uint8_t* fc2_s8 = nullptr;
  // VIT_ACT_F16: the matrices above are float16 copies times 2^e (one e per matrix); the GEMM
  // multiplies its accumulators by these 2^-e
  float qkv_sc = 1.0f, proj_sc = 1.0f, fc1_sc = 1.0f, fc2_sc = 1.0f;
};

struct DeviceWeights {
  void* arena = nullptr;
  size_t bytes = 0;
  const uint16_t* lut = nullptr;     // [3][256] bf16 normalise table
  const uint16_t* pe_w = nullptr;    // [d][kFeatPad]
  std::vector<LayerW> layers;
  const float *mq_g = nullptr, *mq_b = nullptr;
  const uint16_t* m1_w = nullptr; const float* m1_b = nullptr;   // [4d][4d]
  const uint16_t* m2_w = nullptr; const float* m2_b = nullptr;   // [out][4d]
  const uint8_t* m1_w8 = nullptr; const uint8_t* m1_s8 = nullptr;   // VIT_ACT_BF16F8 copies
  const uint8_t* m2_w8 = nullptr; const uint8_t* m2_s8 = nullptr;
  float m1_sc = 1.0f, m2_sc = 1.0f;   // VIT_ACT_F16 weight scales (as in LayerW)
};

}  // namespace vitmi

struct vit_ctx {
  vit_config cfg{};
  int head_dim = 0;
  int mlp_pad = 0;       // mlp_dim rounded up to 64
  int split = 1;         // 2 with hi+lo activation pairs, else 1
  bool f8 = false;       // compensated activations as bf16 + e4m3 residual (VIT_ACT_BF16F8)
  bool f16 = false;      // float16 activations and weight copies (VIT_ACT_F16)
  uint16_t lut[3][256];  // bf16 bits of ((x/255) - mean_c) / std_c, exactly rounded
  bool norm_affine = false;     // fma(x, a_c, b_c) verified equal to lut for every byte
  vitmi::NormAffine affine{};
  std::map<std::string, vitmi::HostTensor> host;
  bool finalized = false;
  int device = -1;
  int n_cu = 0;          // compute units of the device (set at finalize; the planner assumes 256 before)
  vitmi::DeviceWeights w;
  bool is_full_layer(int l) const;
};

struct vit_plan {
  vit_config cfg{};
  int head_dim = 0, mlp_pad = 0, split = 1;
  bool f8 = false;
  int32_t n_items = 0;
  std::vector<int32_t> grid;      // [n][3]
  std::vector<int32_t> nframes;   // [n]
  int64_t n_rows = 0;             // N patches
  int64_t n_units = 0;            // N / 4
  size_t pixel_bytes = 0;
  size_t pixel_read_bytes = 0;    // bytes the patchify reads (an image's frame once, video frames once)
  int32_t max_pos = 0;            // rows of the cos/sin cache
  int32_t nfreq = 0;              // head_dim / 4 frequencies per axis
  int32_t max_seg_full = 0, max_seg_win = 0;
  std::vector<int32_t> row_order; // internal row -> merge-order row

  // metadata blob uploaded to ws at offset 0
  std::vector<uint8_t> meta;
  int64_t off_dims = 0;           // RunDims (always at 0)
  int64_t off_units = 0, off_rowpos = 0, off_unitdst = 0, off_cos = 0, off_sin = 0;
  vitmi::AttnLists full, win;

  // workspace layout (byte offsets; all 256-byte aligned)
  size_t off_x = 0, off_r = 0, off_h = 0, off_q = 0, off_k = 0, off_vt = 0, off_o = 0, off_f = 0;
  size_t off_h8 = 0, off_f8 = 0;  // e4m3 residuals of H and F (VIT_ACT_BF16F8)
  size_t off_o8 = 0;              // e4m3 residual of the attention output O (VIT_ACT_BF16F8)
  size_t off_part = 0;            // partial slots of key-split attention units
  size_t off_pix = 0, off_out = 0, ws_bytes = 0;
  int64_t vt_ld = 0;              // V^T row pitch (tokens), N rounded up to 8
};

struct vit_graph {
  const vit_ctx* ctx = nullptr;
  const vit_plan* plan = nullptr;   // the captured (capacity) plan
  void* ws = nullptr;
  void* graph = nullptr;   // hipGraph_t
  void* exec = nullptr;    // hipGraphExec_t
  bool bucket = false;     // kernels read the batch sizes from the RunDims in ws
  uint8_t* staging = nullptr;   // pinned copy of the metadata region (bucket replays)
  void* staged = nullptr;       // hipEvent_t: the last upload from `staging` has completed
};

namespace vitmi {

// Builds plan metadata and layout (pure host).  Returns VIT_OK or an error.
// key_splits = false: the attention lists keep one unit per query block (no partial slots);
// used for plans whose results are combined with other plans' (the embedding cache's misses).
vit_status build_plan(const vit_ctx* ctx, const int32_t* grid_thw, const int32_t* n_frames,
                      int32_t n_items, vit_plan* p, bool key_splits = true);
// vit_plan_create with the key_splits choice above.
vit_status create_plan(const vit_ctx* ctx, const int32_t* grid_thw, const int32_t* n_frames, int32_t n_items,
                       bool key_splits, vit_plan** out);

// Weight packing + upload (weights.cpp)
vit_status finalize_weights(vit_ctx* ctx, void* stream);
vit_status store_weight(vit_ctx* ctx, const char* name, int32_t dtype, const int64_t* shape,
                        int32_t ndim, const void* host_ptr);

// ---------------------------------------------------------------- kernel launchers

enum GemmEpi : int {
  EPI_F32 = 0,     // out f32 = acc
  EPI_RES = 1,     // out f32 += acc + bias
  EPI_GELU = 2,    // out bf16 = gelu(acc + bias)
  EPI_SWIGLU = 3,  // out bf16 [.][N/2] = silu(gate + bg) * (up + bu), gate/up interleaved per 32 columns
  EPI_QKV = 4,     // RoPE'd q, k -> [heads][rows][head_dim]; v -> [heads][head_dim][rows]
  EPI_OUT = 5,     // out f32 [row_map[m]][n] = acc + bias
};

struct GemmArgs {
  const uint16_t* A = nullptr; int64_t lda = 0;   // blocked (kt_index) [M][lda] bf16, lda >= K (2K split)
  const uint16_t* B = nullptr; int64_t ldb = 0;   // blocked [N][ldb] bf16, ldb >= K
  int M = 0, N = 0, K = 0;                        // K = logical reduction length
  const int32_t* m_dev = nullptr;                 // if set: M read at run time (M above is the capacity)
  // Split activations: when a_group > 0, each A row holds hi/lo pairs in groups of a_group
  // columns, [hi(g) | lo(g)] repeated, and the product is sum_k (hi + lo)[k] * B[n][k].
  int a_group = 0;
  uint32_t a_bytes = 0, b_bytes = 0;              // operand extents (set by launch_gemm)
  int group_m = 8;                                // row tiles per XCD tile group (set by launch_gemm)
  const float* bias = nullptr;
  void* out = nullptr; int64_t ldo = 0;           // fp32 row-major, or blocked bf16 (GELU / SwiGLU)
  // QKV epilogue
  uint16_t* q = nullptr; uint16_t* k = nullptr; uint16_t* vt = nullptr;
  int64_t n_tok = 0;
  int64_t vt_ld = 0;   // V^T row pitch in tokens (a multiple of 8)
  const int32_t* row_pos = nullptr;
  const float* cos_tab = nullptr; const float* sin_tab = nullptr;
  int nfreq = 0, head_dim = 0, hidden = 0;
  float q_scale = 1.0f;   // q is stored multiplied by this (log2(e) / sqrt(head_dim))
  // output scatter
  const int32_t* row_map = nullptr;
  // GELU / SwiGLU: when nonzero, also store lo = bf16(y - bf16(y)) at column + split_off
  int split_off = 0;
  // Compensated activations as bf16 + e4m3 residual (A8 set, a_group 0): the product is
  // sum_k (A[m][k] + 2^-kLoShift A8[m][k]) * B[n][k], the residual term taken against B8 =
  // e4m3(B[n][k] * 2^(127 - b8_scale[n])) with the scaled fp8 MFMA.  K a multiple of 64.
  const uint8_t* A8 = nullptr; int64_t lda8 = 0;   // kt8_index [M][lda8], rows padded to 32
  const uint8_t* B8 = nullptr; int64_t ldb8 = 0;   // kt8_index [N][ldb8]
  const uint8_t* b8_scale = nullptr;               // [N] E8M0 bytes
  uint32_t a8_bytes = 0, b8_bytes = 0;             // (set by launch_gemm)
  // GELU / SwiGLU with A8 mode outputs: the e4m3 residual of each stored activation, times
  // 2^kLoShift, into a kt8_index matrix of ldo8 columns
  uint8_t* out8 = nullptr; int64_t ldo8 = 0;
  // float16 operands (A and B), the f16 MFMA, and float16 activations / q / k / V^T out; the
  // weights carry a power-of-two scale that the accumulators are multiplied by (acc_scale)
  bool f16 = false;
  float acc_scale = 1.0f;
};

vit_status launch_gemm(int epi, const GemmArgs& a, void* stream);
// Raises the dynamic-LDS limit of every GEMM instantiation (call once per process/device).
vit_status prepare_gemm_kernels();

// affine == nullptr: table lookups (always exact)
// n_units_dev (optional): unit count read at run time; n_units is then the capacity.
vit_status launch_normpatch(const uint8_t* pixels, const UnitDesc* units, int64_t n_units,
                            const uint16_t* lut, const NormAffine* affine, uint16_t* x, void* stream,
                            const int32_t* n_units_dev = nullptr);
vit_status launch_normrows_u8(const uint8_t* patches, int64_t n_rows, const uint16_t* lut,
                              uint16_t* x, void* stream);
// Row norm of fp32 rows [rows][d] into bf16 in the blocked GEMM layout; split: each row is
// [hi(d) | lo(d)].  group > 1 stores `group` consecutive rows as one row of group * S * d
// columns (the merger's view of 2x2 patch blocks).
// rows_dev (optional): row count read at run time; rows is then the capacity.
// out8 (instead of split): bf16 rows plus their e4m3 residuals (times 2^kLoShift) in a
// kt8_index matrix of the same view.  f16 (instead of both): float16 rows.
vit_status launch_rownorm(int kind, const float* r, int64_t rows, int d, const float* g,
                          const float* b, float eps, uint16_t* out, bool split, int group,
                          void* stream, const int32_t* rows_dev = nullptr, uint8_t* out8 = nullptr,
                          bool f16 = false);
// Blocked bf16 matrix -> row-major [rows][out_cols] (debug copies): row m of the result is
// row m / group, columns (m % group) * cols + [0, out_cols) of a blocked matrix with
// group * cols columns.
vit_status launch_unblock(const uint16_t* src, int64_t rows, int cols, int group, int out_cols,
                          uint16_t* dst, void* stream);
// Debug copy of a compensated activation in the bf16 + e4m3 form: row m of dst (2 * out_cols
// bf16) = [hi | residual], the residual converted exactly to bf16 (e4m3 value * 2^-kLoShift).
vit_status launch_unblock_f8(const uint16_t* src, const uint8_t* src8, int64_t rows, int cols, int group,
                             int out_cols, uint16_t* dst, void* stream);

struct AttnArgs {
  const uint16_t* q = nullptr; const uint16_t* k = nullptr; const uint16_t* vt = nullptr;
  // output in the blocked GEMM layout: hi = bf16(o) rows of o_ld columns; with o_split the
  // row is [hi(hidden) | lo(hidden)] (o_ld = 2 * hidden, lo = bf16(o - hi)); with o8 the
  // e4m3 residual (o - hi) * 2^kLoShift goes to a kt8_index matrix of hidden columns
  uint16_t* o = nullptr;
  bool o_split = false;
  uint8_t* o8 = nullptr;
  bool f16 = false;   // q, k, V^T and the output are float16 (else bfloat16)
  int64_t n_tok = 0;
  int64_t vt_ld = 0;   // V^T row pitch in tokens: a multiple of 8, pad columns finite (zero)
  int heads = 0, head_dim = 0;
  const AttnWork* work_long = nullptr; int n_long = 0;
  const AttnWork* work_short = nullptr; int n_short = 0;
  // if set: list lengths read at run time (n_long / n_short above are the capacities)
  const int32_t* n_long_dev = nullptr; const int32_t* n_short_dev = nullptr;
  // partial slots of key-split units: [heads][n_parts][head_dim + 2][256] floats (rows: the
  // unnormalised output dims, then the running offset m, then the denominator l; 256 queries)
  float* part = nullptr; int n_parts = 0;
};
vit_status launch_attention(const AttnArgs& a, void* stream);
// Combines the partial slots of each merge into the output (same layout and forms as the
// attention output).
vit_status launch_attention_merge(const AttnArgs& a, const AttnMerge* merge, int n_merge, void* stream);
// Per-item partial sums of the pixel content key (pixel_hash.hip): items_dev[i] = {byte offset,
// 64-bit word count}, sums_dev[2 i + j] = lane-j sum (zeroed here first).
vit_status launch_pixel_hash(const uint8_t* pixels, const int64_t* items_dev, int n_items, int64_t max_words,
                             uint64_t* sums_dev, void* stream);
// Device resize of uint8 HWC frames to the 28-pixel grid (resize.hip); resize_side gives the
// target of one side.
int resize_side(int s);
vit_status launch_resize(const uint8_t* src, int sh, int sw, int frames, uint8_t* dst, int dh, int dw,
                         void* stream);
// The checks every encode entry point makes on (ctx, plan, workspace).
vit_status check_plan_ws(const vit_ctx* ctx, const vit_plan* plan, const void* ws, size_t ws_bytes);
// Zeroes V^T columns [n_tok, n_tok + 64), clipped to the pitch, of every row (the attention
// reads whole 16-byte chunks up to 40 keys past a segment; those keys get probability 0 and
// must not be NaN).  n_tok_dev (optional): token count read at run time.
vit_status launch_vt_pad_zero(uint16_t* vt, int rows, int64_t n_tok, int64_t vt_ld, void* stream,
                              const int32_t* n_tok_dev = nullptr);

}  // namespace vitmi
