/*
 * vit.h -- C ABI of the MI355X (gfx950) vision-tower library.
 *
 * The library runs the Qwen2-VL / Qwen2.5-VL-style vision tower forward over
 * packed variable-resolution images and videos on one GPU:
 *
 *   uint8 pixels -> rescale/normalise + patchify -> patch-embed GEMM
 *   -> L x [norm -> QKV GEMM + 2D RoPE -> block-diagonal attention
 *           -> out-proj + residual -> norm -> MLP + residual]
 *   -> 2x2 patch merger MLP -> embeddings.
 *
 * Sources for what each step computes (pages, not code):
 *  - vLLM PR #55370 report ("Make mm_device_do_normalize encoder-cudagraph
 *    safe"), implementation breakdown and review highlights: the tower owns
 *    the rescale + normalise of integer pixels as its first step, so eager and
 *    graph-replayed forwards both normalise exactly once; uint8 values are
 *    exact in bfloat16.
 *  - "vLLM multimodal inference | ViT performance optimisation" (blog):
 *    section 2.2 (patchify in merge-unit order, flatten_patches, patch
 *    embedding, 2D RoPE, encoder, patch merger), 3.2 (patch embedding is a
 *    stride = kernel 3D conv done as one GEMM), 3.3 (cos/sin cache, 2D
 *    positions, first half of the angles from the row position, second half
 *    from the column position, window-attention order), 3.4 (cu_seqlens
 *    computed once per forward, uploaded asynchronously, shared by every
 *    layer; attention never crosses an item boundary), 3.5 (fused norm/RoPE/
 *    activation kernels to cut launches).
 *  - "GPUModelRunner.execute_model" notes, limits section: an empty batch
 *    runs no forward; graphs are captured against a fixed workspace.
 *
 * Conventions
 *  - Every call returns vit_status (VIT_OK == 0) unless noted.  On failure
 *    nothing has been enqueued and vit_last_error() describes the problem.
 *  - All validation happens before the first enqueue.
 *  - The caller owns every device buffer (pixels, workspace, output).  The
 *    library owns its weight arena (inside vit_ctx) and the plan's host data.
 *    Only vit_finalize_weights and vit_graph_capture[_bucket] allocate device
 *    memory (graph objects); vit_graph_capture_bucket also allocates pinned
 *    host memory for its staging buffer.  The embedding cache's arena is the
 *    caller's.
 *  - Device pointers are plain HIP device addresses; streams are hipStream_t
 *    passed as void* (NULL = the default stream).
 *  - Pixels are uint8 only: there is no float input and no "already
 *    normalised" mode, so un-normalised and doubly-normalised inputs cannot
 *    be expressed.
 *  - A finalized vit_ctx is read-only: concurrent vit_encode calls on
 *    distinct workspaces are allowed.  Two calls sharing a workspace race.
 */
#ifndef VIT_H_
#define VIT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vit_status;
#define VIT_OK           0
#define VIT_E_ARG        1  /* bad argument (null pointer, bad enum, bad config value) */
#define VIT_E_SHAPE      2  /* bad grid_thw / n_frames / tensor shape */
#define VIT_E_WEIGHTS    3  /* unknown, duplicate, missing or mis-shaped weight */
#define VIT_E_WORKSPACE  4  /* workspace or destination buffer too small */
#define VIT_E_STATE      5  /* call out of order (e.g. encode before finalize) */
#define VIT_E_HIP        6  /* HIP runtime error (asynchronous faults surface here) */

#define VIT_MLP_GELU     0  /* fc1 -> exact-erf GELU -> fc2 */
#define VIT_MLP_SWIGLU   1  /* SiLU(gate) * up -> down */
#define VIT_NORM_LAYER   0  /* LayerNorm with gain and shift, biased variance */
#define VIT_NORM_RMS     1  /* RMSNorm with gain */
#define VIT_F32          0
#define VIT_BF16         1

#define VIT_ACT_BF16     0  /* GEMM activation operands rounded once to bfloat16 */
#define VIT_ACT_BF16X2   1  /* norm, MLP and merger activations kept as hi+lo bfloat16 pairs */
#define VIT_ACT_BF16F8   2  /* the same activations kept as bfloat16 + e4m3 residual */
#define VIT_ACT_F16      3  /* every GEMM / attention activation in float16 (the default form) */

#define VIT_MAX_FULL_LAYERS 64

/* Tower hyper-parameters.  Fixed by this library: patch 14, temporal_patch 2,
 * merge 2 (checked).  hidden % 64 == 0, head_dim = hidden / heads must be 32,
 * 64 or 80 (80 is the Qwen2-VL head size), layers >= 0. */
typedef struct vit_config {
  int32_t hidden;
  int32_t heads;
  int32_t layers;
  int32_t mlp_dim;          /* fc1 width (GELU) or gate/up width (SwiGLU) */
  int32_t mlp_kind;         /* VIT_MLP_* */
  int32_t norm_kind;        /* VIT_NORM_* (blocks and merger) */
  float   norm_eps;         /* 1e-6 */
  int32_t patch;            /* 14 */
  int32_t temporal_patch;   /* 2 */
  int32_t merge;            /* 2 */
  int32_t out_dim;          /* merger output width */
  float   rope_theta;       /* 10000 */
  float   mean[3];          /* per-channel mean of x/255, RGB */
  float   std[3];           /* per-channel std, > 0 */
  int32_t window_px;        /* 0: no window attention; else window side in pixels (multiple of 28) */
  int32_t n_full_attn_layers;
  int32_t full_attn_layers[VIT_MAX_FULL_LAYERS]; /* 0-based layers that attend over whole items */
  /* VIT_ACT_BF16X2: each norm output, attention output, MLP activation and merger
   * activation x is stored as hi = bf16(x), lo = bf16(x - hi) and the GEMM that consumes it
   * runs over both halves against the same bf16 weights (twice the MFMA work of those
   * products), which removes their activation rounding; q, k, v and the attention
   * probabilities stay single bf16.  VIT_ACT_BF16F8 keeps the same activations as
   * hi = bf16(x) plus the residual x - hi in OCP e4m3 (scaled by 2^9); the GEMM adds the
   * residual's product against an e4m3 copy of the weights (per-row power-of-two scales)
   * through the scaled fp8 MFMA, so the residual costs half the MFMA time of a second bf16
   * product and 1 instead of 2 bytes per element (its error, ~2^-12 of x, stays far below
   * the bf16 rounding it compensates).  VIT_ACT_BF16 rounds every GEMM activation once.
   * VIT_ACT_F16 (recommended) stores every GEMM and attention activation -- norm outputs,
   * q, k, v, the attention probabilities and output, MLP and merger activations -- in IEEE
   * float16, rounded once (relative error 2^-12, the compensated forms' level, with no
   * second product), and multiplies them on the float16 MFMA (the bf16 rate) against float16
   * copies of the weights: each matrix's bf16 values times one power of two, exact for every
   * weight above 2^-39 of the matrix's largest.  Only the patch embedding stays bf16 (its
   * input, the normalised pixels, is bf16 by definition). */
  int32_t activation_precision;
} vit_config;

typedef struct vit_ctx vit_ctx;
typedef struct vit_plan vit_plan;
typedef struct vit_graph vit_graph;
typedef struct vit_cache vit_cache;

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* vit_last_error(void);

/* Validates cfg and builds the exact normalise table on the host.  No GPU call.
 * Defined by: "vLLM multimodal inference | ViT performance optimisation",
 * section 2.2 (patch size, temporal patch, merge size, encoder and patch
 * merger) and section 3.3 (2D RoPE base, window-attention layers); vLLM PR
 * #55370 report, implementation breakdown item 1 (the normaliser's rescale,
 * mean and std are parameters of the tower, injected at construction).
 * Errors: VIT_E_ARG for a NULL pointer or any out-of-range field; *out is
 * NULL then.  The caller releases the context with vit_destroy. */
vit_status vit_create(const vit_config* cfg, vit_ctx** out);

/* Copies one host tensor into the context (host buffer may be freed after
 * the call).  Defined by: vLLM PR #55370 report, key code (the tower's
 * stacked-parameter mapping loads separate q, k, v projections into one qkv
 * matrix) and "vLLM multimodal inference | ViT performance optimisation",
 * section 3.2 (the patch-embedding conv weight reshaped to a 2D matrix).
 * Errors: VIT_E_WEIGHTS for a duplicate name, VIT_E_SHAPE for a non-positive
 * dimension, VIT_E_STATE after vit_finalize_weights, VIT_E_ARG for a NULL
 * pointer or a dtype other than VIT_F32 / VIT_BF16 (bf16 given as raw uint16
 * bits).  Names and shapes are checked against the tower by
 * vit_finalize_weights.
 * Canonical names and shapes ([out, in] for linears):
 *   pe.w [hidden][3][2][14][14] (or [hidden][1176])
 *   blk{l}.n1.g, blk{l}.n1.b (LayerNorm only), blk{l}.n2.g, blk{l}.n2.b  [hidden]
 *   blk{l}.qkv.w [3*hidden][hidden], blk{l}.qkv.b [3*hidden]
 *     (or split blk{l}.q.w/.b, blk{l}.k.w/.b, blk{l}.v.w/.b, stacked q;k;v)
 *   blk{l}.proj.w [hidden][hidden], blk{l}.proj.b [hidden]
 *   GELU:   blk{l}.fc1.w [mlp][hidden], .b; blk{l}.fc2.w [hidden][mlp], .b
 *   SwiGLU: blk{l}.gate.w, blk{l}.up.w [mlp][hidden], .b; blk{l}.down.w [hidden][mlp], .b
 *   mrg.nq.g, mrg.nq.b (LayerNorm only) [hidden]
 *   mrg.fc1.w [4h][4h], mrg.fc1.b [4h]; mrg.fc2.w [out][4h], mrg.fc2.b [out]
 * dtype VIT_F32 values are rounded to bfloat16 (nearest, ties to even) for
 * matrices; norm parameters and biases are kept in float32. */
vit_status vit_load_weight(vit_ctx* ctx, const char* name, int32_t dtype, const int64_t* shape,
                           int32_t ndim, const void* host_ptr);

/* Checks completeness, packs (q/k/v stacking, RoPE pair order, K padding,
 * gate/up interleave) and uploads the weights into a device arena owned by
 * ctx.  Synchronises `stream` before returning.  ctx is read-only afterwards.
 * Defined by: the same passages as vit_load_weight.  Errors: VIT_E_WEIGHTS
 * names the first missing, unknown or mis-shaped tensor; VIT_E_HIP if the
 * arena cannot be allocated or uploaded; VIT_E_STATE if called twice. */
vit_status vit_finalize_weights(vit_ctx* ctx, void* stream);

/* Pure host: validates the batch and builds every piece of per-forward
 * metadata (cu_seqlens, merge-ordered positions, window order, attention
 * work lists, RoPE cos/sin cache, workspace layout).  Defined by: "vLLM
 * multimodal inference | ViT performance optimisation", section 2.2
 * (grid_thw records each item's patch counts), section 3.3 (positions from
 * grid_thw, cos/sin cache, window-attention order) and section 3.4
 * (cu_seqlens built once per forward and shared by every layer).
 * Errors (nothing allocated on the device, *out NULL): VIT_E_SHAPE for a bad
 * (t, h, w) / n_frames pair, a side above 16384 patches, more than 2^28
 * patches, a video frame of 2^31 bytes or more, or a batch whose largest
 * device operand (normalised patches, norm output, MLP activation, merger
 * views, their e4m3 residuals, per-head q / k / V^T) would reach 2 GiB
 * (32-bit buffer addressing); VIT_E_ARG for NULL pointers.
 *   grid_thw [n_items][3] = (t, h, w) in patches; h, w even, t >= 1.
 *   n_frames [n_items]: 1 for an image (t must be 1; the frame is used for
 *     both temporal slots), or 2*t for a video.
 * n_items == 0 is allowed: encode is then a no-op. */
vit_status vit_plan_create(const vit_ctx* ctx, const int32_t* grid_thw, const int32_t* n_frames,
                           int32_t n_items, vit_plan** out);
void vit_plan_destroy(vit_plan* plan);

/* Sizes of a plan ("vLLM multimodal inference | ViT performance
 * optimisation", section 2.2: every 2x2 merge unit becomes one output token).
 * pixel_bytes = sum over items of n_frames*H*W*3 (H = 14h, W = 14w);
 * ws_bytes = workspace the plan needs; out_rows = N/4 merged tokens;
 * out_cols = out_dim.  Any output pointer may be NULL. */
vit_status vit_plan_sizes(const vit_plan* plan, size_t* pixel_bytes, size_t* ws_bytes,
                          int64_t* out_rows, int64_t* out_cols);

/* Number of patches N and the library's internal row order: dst[i] = the
 * merge-order row index of internal row i (identity unless window attention
 * reorders rows).  dst may be NULL; otherwise it holds N int32 (host). */
vit_status vit_plan_rows(const vit_plan* plan, int64_t* n_patches, int32_t* dst);

/* The long attention work units of a plan (test and tuning aid; pure host).
 * Segments are the block-diagonal attention's per-item (or per-window)
 * sequences ("vLLM multimodal inference | ViT performance optimisation",
 * section 3.4, cu_seqlens).  layer_kind 0 = item segments, 1 = windows.
 * split 0: the plain list (one unit per block of 256 queries of a segment;
 * what bucketed graphs run); split 1: the list the eager forward and
 * whole-forward graphs run (the plain list, or key-split units when the
 * planner split some units' key ranges to balance the launch's tail, in
 * which case *n_merge > 0 query blocks are merged from *n_parts partial
 * slots).  units, if not NULL, receives *n_units rows of 8 int32 (host):
 * segment start row, segment length, first query of the unit (relative to
 * the segment start), first and end key block (32 keys each), partial slot
 * (-1: the unit covers all keys of its queries), 0, 0.  Call once with
 * units = NULL to size the buffer.  Errors: VIT_E_ARG for a NULL plan or a
 * layer_kind / split outside {0, 1}. */
vit_status vit_plan_attention_units(const vit_plan* plan, int32_t layer_kind, int32_t split,
                                    int32_t* units, int32_t* n_units, int32_t* n_merge, int32_t* n_parts);

/* Enqueues the whole forward on `stream` and returns without synchronising.
 * Defined by: "vLLM multimodal inference | ViT performance optimisation",
 * section 2.2 (encoding steps 1-4: patchify, patch embedding, 2D RoPE,
 * encoder, patch merger); vLLM PR #55370 report, implementation breakdown
 * items 1-2 (rescale + normalise of integer pixels is the tower's own first
 * step, so every path normalises exactly once); "GPUModelRunner.execute_model"
 * notes (an empty batch runs no forward).  Errors: VIT_E_STATE before
 * vit_finalize_weights; VIT_E_ARG for a plan of another configuration, NULL
 * pixels / out with patches to encode, or an unaligned workspace;
 * VIT_E_WORKSPACE if ws_bytes is too small; VIT_E_HIP for a launch failure
 * (earlier asynchronous faults also surface here).  A plan with no items
 * returns VIT_OK and enqueues nothing (ws, pixels and out may then be NULL).
 *   pixels_u8: device, pixel_bytes; items in order, each n_frames frames of
 *              H x W x 3 uint8, HWC, RGB, row-major.
 *   ws:        device, >= ws_bytes, 256-byte aligned; contents are scratch.
 *   out:       device float32 [N/4][out_dim], merged tokens in item order. */
vit_status vit_encode(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8, void* ws,
                      size_t ws_bytes, float* out, void* stream);

/* Size of the static device scratch that vit_encode_noalloc uses as its workspace. */
#define VIT_NOALLOC_SCRATCH_BYTES (64u << 20)

/* vit_encode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same forward, same kernels, same
 * arguments minus the workspace: the workspace is a static device array of
 * VIT_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU, held until the process
 * ends; the call allocates nothing.  Enough for a plan whose ws_bytes (vit_plan_sizes) fit:
 * for a 1280-wide tower with a 5120-wide MLP, about 1600 patches (a 448 x 448 image needs
 * 40 MiB).  Errors as vit_encode, plus VIT_E_WORKSPACE when the plan needs more than the
 * scratch (nothing is enqueued) and VIT_E_STATE when the current device is not the one the
 * weights were uploaded to.  Every call on a GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU race, so issue them on one stream or order them. */
vit_status vit_encode_noalloc(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8,
                              float* out, void* stream);

/* Same forward from uint8 flatten_patches instead of frames (the pages' own
 * tower input: vLLM PR #55370 report, implementation breakdown item 2 and
 * review highlights -- the tower receives integer pixels already cut into
 * flatten_patches; "vLLM multimodal inference | ViT performance
 * optimisation", sections 2.2 and 3.2).  Errors as vit_encode, plus VIT_E_ARG
 * for a patches pointer that is not 8-byte aligned:
 *   patches_u8: device [N][1176] uint8 rows in merge order, features
 *   (channel, temporal slot, row, column). */
vit_status vit_encode_patches_u8(const vit_ctx* ctx, const vit_plan* plan,
                                 const uint8_t* patches_u8, void* ws, size_t ws_bytes, float* out,
                                 void* stream);

/* Captures the whole forward (normalisation included) into a HIP graph that
 * reads pixels from, and writes the output into, regions inside `ws`
 * (see vit_graph_io).  The plan's metadata is uploaded into ws before the
 * capture begins; the graph is bound to (ctx, plan, ws).  Defined by: vLLM
 * PR #55370 report, implementation breakdown item 2 (normalisation captured
 * with the encoder graph, the same call chain as eager) and review
 * highlights item 3 (a uint8 graph input buffer: no per-replay cast);
 * "GPUModelRunner.execute_model" notes, key files (graphs captured once at
 * start against a locked workspace).  Errors as vit_encode; VIT_E_SHAPE for
 * an empty plan; VIT_E_HIP if capture or instantiation fails.  The caller
 * releases the graph with vit_graph_destroy before freeing ws. */
vit_status vit_graph_capture(const vit_ctx* ctx, const vit_plan* plan, void* ws, size_t ws_bytes,
                             void* stream, vit_graph** out);
/* Device addresses of the graph's uint8 pixel input (pixel_bytes) and
 * float32 output ([N/4][out_dim]) regions (same passages as
 * vit_graph_capture).  Either output pointer may be NULL. */
vit_status vit_graph_io(const vit_graph* g, uint8_t** pixels_in, float** out);
/* Replays the captured forward on `stream` (asynchronous).  Replays of one
 * graph share its workspace: issue them on one stream.  VIT_E_HIP if the
 * launch fails. */
vit_status vit_graph_launch(vit_graph* g, void* stream);
void vit_graph_destroy(vit_graph* g);

/* Shape-bucketed graph ("GPUModelRunner.execute_model" notes, capture
 * section: graphs are captured largest shape first and smaller ones reuse
 * the memory; vLLM PR #55370 report, comment highlights: a u8 input buffer
 * inside the graph, and no normalisation work on padding rows).
 * vit_graph_capture_bucket captures the forward for a capacity plan
 * (`plan`: the largest batch the graph must serve) in a form whose kernels
 * read the batch sizes (patches, merge units, attention work-list lengths)
 * from device memory, so padded capacity is skipped by normalisation,
 * attention and the products rather than computed.  Launched plainly
 * (vit_graph_launch) it encodes `plan`.  Its attention runs the plain work
 * lists (one unit per 256-query block, see vit_plan_attention_units), never
 * key-split units, so for a plan whose eager forward splits key ranges the
 * replay equals vit_encode's result to rounding (the same softmax summed in
 * another order) rather than bit for bit.  Also allocates one pinned host
 * staging buffer of the plan's metadata size.  Same requirements as
 * vit_graph_capture. */
vit_status vit_graph_capture_bucket(const vit_ctx* ctx, const vit_plan* plan, void* ws,
                                    size_t ws_bytes, void* stream, vit_graph** out);
/* Replays a bucketed graph for another plan of the same context: the plan's
 * metadata is written into the graph's metadata region (one asynchronous
 * host-to-device copy on `stream`, from the staging buffer, which is reused
 * once the previous copy has completed) and the graph is launched.  The
 * caller writes the plan's pixels (its pixel_bytes) at vit_graph_io's input
 * first; its output is rows [0, N/4) of vit_graph_io's output.  The plan
 * must fit the capacity: patches, pixel bytes, largest grid side and each
 * attention work-list length at most the captured plan's (VIT_E_SHAPE names
 * the first that does not), and the same tower configuration (VIT_E_ARG).
 * VIT_E_STATE for a graph not captured with vit_graph_capture_bucket.  An
 * empty plan enqueues nothing.  Replays of one graph share its workspace:
 * issue them on one stream (or order them), as for vit_graph_launch. */
vit_status vit_graph_launch_plan(vit_graph* g, const vit_plan* plan, void* stream);

/* Vision-embedding cache ("vLLM multimodal inference | ViT performance
 * optimisation", section 2.3: a vision-embedding cache shared across
 * requests).  Trusted input only: a hit is decided by the 128-bit content
 * key (vit_pixel_keys) without comparing pixel bytes, and that key is not
 * collision resistant against a deliberate search, so a cache shared between
 * mutually untrusting clients could be fed crafted colliding pixels.  Merged embeddings of items are kept in `arena` (device,
 * caller-owned, 256-byte aligned, arena_bytes may be 0) and reused when an
 * item with the same pixel content key and the same grid (t, h, w, n_frames)
 * is encoded again through vit_encode_cached.  The arena is a ring with
 * first-in first-out eviction; an item larger than the arena is never cached.
 * The cache is bound to ctx (the weights).  No GPU call; not thread-safe. */
vit_status vit_cache_create(const vit_ctx* ctx, void* arena, size_t arena_bytes, vit_cache** out);
/* Number of cached items and arena bytes they hold. */
vit_status vit_cache_stats(const vit_cache* cache, int64_t* entries, size_t* bytes_used);
void vit_cache_destroy(vit_cache* cache);
/* vit_encode through the cache: computes every item's pixel content key on
 * the device, copies the keys to the host and synchronises `stream` (the
 * hit/miss split is a host decision), copies cached items' rows from the
 * arena into `out`, encodes the remaining items as one batch (their pixels
 * gathered into the workspace; that batch runs no key-split attention units,
 * so an item's cached rows do not depend on which items missed with it),
 * writes their rows into `out` (item order, as vit_encode) and caches them.
 * The rows equal vit_encode's for the same batch bit for bit when that
 * batch's plan runs no key-split units (vit_plan_attention_units), and to
 * rounding otherwise.  Everything after the key read is
 * asynchronous on `stream`; the arena must not be touched by other work
 * until it completes.  *n_hits (optional) receives the number of items
 * served from the cache.  pixels_u8 must be 16-byte aligned.  Errors as
 * vit_encode. */
vit_status vit_encode_cached(const vit_ctx* ctx, vit_cache* cache, const vit_plan* plan,
                             const uint8_t* pixels_u8, void* ws, size_t ws_bytes, float* out,
                             void* stream, int32_t* n_hits);
/* The content keys alone: keys[2 i], keys[2 i + 1] (host array of 2 * n_items)
 * receive item i's 128-bit key.  With the item's pixel bytes read as L / 8
 * little-endian 64-bit words w_k, lane j (G_0 = 0x9e3779b97f4a7c15,
 * G_1 = 0xd1b54a32d192ed03) is mix(S_j ^ (L * G_j)) with
 * S_j = sum_k mix(w_k + (k + 1) G_j) mod 2^64 and mix the SplitMix64
 * finaliser (Steele, Lea and Flood, OOPSLA 2014).  A content key, not a
 * cryptographic hash.  Synchronises `stream`. */
vit_status vit_pixel_keys(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8,
                          void* ws, size_t ws_bytes, uint64_t* keys, void* stream);

/* Device resize before the path ("vLLM multimodal inference | ViT
 * performance optimisation", section 2.2: the preprocessor resizes and pads
 * images; SGLang PR #35349 report: CPU preprocessing caps serving
 * throughput).  vit_resize_side(s) = the nearest multiple of 28 to s (half
 * up), at least 28 (0 for s < 1).  vit_resize_u8 resizes `frames` HWC RGB
 * uint8 frames of sh x sw pixels (device, back to back) to
 * vit_resize_side(sh) x vit_resize_side(sw) into dst (device, same layout;
 * dst_bytes must cover it, VIT_E_WORKSPACE otherwise; src and dst 4-byte
 * aligned and not overlapping): bilinear with half-pixel centres (source coordinate
 * (d + 0.5) * S / D - 0.5, clamped), 11-bit fixed-point weights in integer
 * arithmetic, rounded half up, so results are exact.  Asynchronous on
 * `stream`; no allocation.  Sides up to 8192 pixels and sources under
 * 4 GiB (VIT_E_SHAPE otherwise).  The output frames are valid vit_encode input for
 * grid (t, vit_resize_side(sh) / 14, vit_resize_side(sw) / 14). */
int32_t vit_resize_side(int32_t pixels);
vit_status vit_resize_u8(const uint8_t* src, int32_t sh, int32_t sw, int32_t frames, uint8_t* dst,
                         size_t dst_bytes, void* stream);

void vit_destroy(vit_ctx* ctx);

/* Per-kernel timing of one forward.  One record per kernel class (e.g.
 * "gemm_qkv_rope", "attention"); `flops` counts algorithmic MFMA work
 * (2 per multiply-add, unpadded shapes; attention 4*hidden*sum(len^2)) and
 * `bytes` algorithmic HBM traffic of memory-bound kernels, both summed over
 * the class's launches. */
typedef struct vit_kernel_stat {
  char    name[32];
  int32_t launches;
  int32_t mfma_bound;   /* 1: rated against the MFMA peak, 0: against HBM bandwidth */
  double  total_ms;     /* sum of hipEvent-measured launch durations */
  double  flops;
  double  bytes;
} vit_kernel_stat;

/* vit_encode with hipEvents recorded around every kernel launch on `stream`.
 * Synchronises `stream` before returning and writes up to max_stats records
 * into stats (host array); *n_stats receives the number of classes. */
vit_status vit_encode_profiled(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8,
                               void* ws, size_t ws_bytes, float* out, void* stream,
                               vit_kernel_stat* stats, int32_t max_stats, int32_t* n_stats);

/* Test hook: runs the forward up to one intermediate and copies it to `dst`
 * (device), in internal row order.
 *   layer = -1: step 0 normalised patches bf16 [N][1176];
 *               step 1 patch embedding f32 [N][hidden]
 *   0 <= layer < layers:
 *               1 norm1 bf16 [N][S*hidden];
 *               2 q after RoPE, times log2(e)/sqrt(head_dim) (the scale the attention
 *                 kernel expects, applied before rounding), bf16 [heads][N][head_dim];
 *               3 k bf16 [heads][N][head_dim]; 4 v bf16 [heads][head_dim][N];
 *               5 attention bf16 [N][S*hidden]; 6 residual after out-proj f32 [N][hidden];
 *               7 norm2 bf16 [N][S*hidden]; 8 MLP activation bf16 [N][S*mlp_pad];
 *               9 block output f32 [N][hidden]
 *   layer = layers: 1 merger norm bf16 [N][S*hidden]; 2 merger hidden bf16 [N/4][S*4*hidden];
 *               3 output f32 [N/4][out_dim] (item order)
 * where S = 2 with VIT_ACT_BF16X2 and VIT_ACT_BF16F8 (each row holds hi then lo
 * halves, the e4m3 residual converted exactly to bfloat16; for the merger norm
 * each patch row is [hi | lo]) and 1 otherwise, and mlp_pad is
 * mlp_dim rounded up to a multiple of 64 (columns past mlp_dim are zero).
 * dst_bytes must cover the tensor; VIT_E_WORKSPACE otherwise. */
vit_status vit_debug_stage(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8,
                           void* ws, size_t ws_bytes, int32_t layer, int32_t step, void* dst,
                           size_t dst_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VIT_H_ */
