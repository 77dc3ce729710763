// normpatch: uint8 HWC frames -> bfloat16 flatten_patches rows, in one pass.
//
// The tower's first step rescales and normalises integer pixels into the
// tower dtype (vLLM PR #55370 report, implementation breakdown); patchify
// cuts 14x14 patches over two temporal slots, keeps each 2x2 merge unit's
// rows adjacent and flattens features in (channel, slot, row, column) order
// ("vLLM multimodal inference | ViT performance optimisation", sections 2.2
// and 3.2).  The normalised value of every (channel, byte) pair is taken from
// a 3x256 table of exactly rounded bfloat16 values, so the result is the
// correctly rounded quotient bit for bit; when the library has verified on the
// host that one float32 fma per byte rounds to the same 768 values, the
// kernel evaluates that fma instead of the table (fewer LDS lookups).
//
// HBM-bound streaming kernel.  One workgroup of 512 threads handles
// kUnitsPerBlock = 4 merge units that are consecutive in row order, so both
// sides stream:
//  * input: each unit's 28 pixel rows x 84 bytes per temporal slot are staged
//    in LDS with 12-byte loads ordered (slot, pixel row, unit, piece), so
//    adjacent lanes read adjacent bytes of one image row, all issued before
//    the first LDS store, and the block's tables are built while they are in
//    flight; an image's single frame is read once and serves both temporal
//    slots;
//  * output: the block's 4 * kUnitsPerBlock = 16 rows of 1184 bf16 (columns
//    1176..1183 zero, so the patch-embed GEMM needs no K tail) are one whole
//    16-row group of the blocked GEMM layout (kt_index), i.e. one contiguous
//    run, written as 16-byte nontemporal stores by consecutive lanes in
//    memory order.
// (On the 1.3 GB streaming batch, 4 units per 512-thread workgroup with the
// loads issued first measured 224-228 us against 236-238 us for 8 units with
// the tables built first; 16 units, or 128- and 1024-thread workgroups, were
// slower.)
// Two tables built at compile time (video units, image units) map each output
// feature to its staged byte, so a 16-byte output chunk costs one table read
// and 8 byte lookups, with no per-element index arithmetic.
#include <hip/hip_runtime.h>

#include "vit_internal.h"

namespace vitmi {

namespace {

constexpr int kThreads = 512;
constexpr int kUnitsPerBlock = 4;
constexpr int kRowBytes = kUnitPx * 3;                        // 84 bytes of one unit pixel row
constexpr int kRowDwords = kRowBytes / 4;                     // 21
constexpr int kSlotBytes = kUnitPx * kRowBytes;               // 2352 bytes of one temporal slot
constexpr int kUnitBytes = kTemporal * kSlotBytes;            // 4704
constexpr int kUnitDwords = kUnitBytes / 4;                   // 1176
constexpr int kChunksPerRow = kFeatPad / 8;                   // 148
constexpr int kChunksPerUnit = 4 * kChunksPerRow;             // 592
constexpr int kColBlocks = kFeatPad / 32;                     // 37 blocks of 32 features
static_assert(4 * kUnitsPerBlock % 16 == 0, "a block's rows are whole 16-row groups");
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
constexpr int kRowPieces = kRowBytes / 12;                    // 7 pieces of 12 bytes per unit row
constexpr int kPieceIds = kUnitsPerBlock * kTemporal * kUnitPx * kRowPieces;
constexpr int kLoadsPerThread = (kPieceIds + kThreads - 1) / kThreads;

// 12 bytes of a pixel row (4-byte aligned: unit rows start at multiples of 84 bytes)
struct alignas(4) Piece {
  uint32_t a, b, c;
};

static_assert(kFeatPad % 8 == 0 && kFeatPad >= kFeat, "row padding");

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Staged byte of every output feature, one table per kind of unit: feature
// f = ((c * 2 + tau) * 14 + i) * 14 + j of the unit's top-left patch is byte
// (tau * 28 + i) * 84 + 3 * j + c of a video unit's two staged frames, and byte
// i * 84 + 3 * j + c of an image unit's one frame (both temporal slots are that
// frame).  Pad features (>= 1176) are whole chunks and never read.  Built at
// compile time; each workgroup copies both tables into LDS.
struct FeatureTables {
  uint16_t off[2][kFeatPad];   // [0] video unit, [1] image unit
  constexpr FeatureTables() : off() {
    for (int f = 0; f < kFeatPad; ++f) {
      if (f >= kFeat) continue;
      const int c = f / 392, r1 = f - c * 392;
      const int tau = r1 / 196, r2 = r1 - tau * 196;
      const int i = r2 / 14, j = r2 - i * 14;
      off[0][f] = (uint16_t)((tau * kUnitPx + i) * kRowBytes + 3 * j + c);
      off[1][f] = (uint16_t)(i * kRowBytes + 3 * j + c);
    }
  }
};
__constant__ __attribute__((aligned(16))) FeatureTables g_feat = FeatureTables();
constexpr int kPadChunk = kFeat / 8;   // first chunk of pad features (147)
constexpr int kChanChunks = 392 / 8;   // chunks per channel (49)

template <bool AFFINE>
__global__ void __launch_bounds__(kThreads)
normpatch_kernel(const uint8_t* __restrict__ pixels, const UnitDesc* __restrict__ units,
                 int64_t n_units, const int32_t* __restrict__ n_units_dev, const uint16_t* __restrict__ lut_g,
                 NormAffine na, uint16_t* __restrict__ x) {
  __shared__ uint32_t stage[kUnitsPerBlock * kUnitDwords];
  __shared__ __attribute__((aligned(16))) uint16_t tab[2 * kFeatPad];
  __shared__ uint16_t lut[3 * 256];
  __shared__ UnitDesc sud[kUnitsPerBlock];
  const int tid = threadIdx.x;
  const int64_t u0 = (int64_t)blockIdx.x * kUnitsPerBlock;
  const int64_t n_all = n_units_dev ? (int64_t)*n_units_dev : n_units;   // run-time count (bucketed graph)
  if (u0 >= n_all) return;
  const int nu = (int)min<int64_t>(kUnitsPerBlock, n_all - u0);
  if (tid < nu) sud[tid] = units[u0 + tid];
  __syncthreads();

  // stage: piece id -> (slot, pixel row, unit, 12-byte piece of the row); images skip slot 1.
  // Every load of the block is issued before the first LDS store, and the block's tables are
  // built while those loads are in flight, so a thread waits for one memory latency.
  Piece v[kLoadsPerThread];
  int dst[kLoadsPerThread];
#pragma unroll
  for (int k = 0; k < kLoadsPerThread; ++k) {
    const int id = tid + k * kThreads;
    const int pc = id % kRowPieces, t = id / kRowPieces;
    const int u = t % kUnitsPerBlock, rest = t / kUnitsPerBlock;
    const int row = rest % kUnitPx, slot = rest / kUnitPx;
    dst[k] = -1;
    if (id < kPieceIds && u < nu && !(slot == 1 && sud[u].fstride == 0)) {
      const UnitDesc ud = sud[u];
      const uint8_t* src = pixels + ud.px_off + (int64_t)slot * ud.fstride + (int64_t)row * ud.pitch + 12 * pc;
      v[k] = *reinterpret_cast<const Piece*>(src);
      dst[k] = u * kUnitDwords + (slot * kUnitPx + row) * kRowDwords + 3 * pc;
    }
  }
  if (!AFFINE)
    for (int i = tid; i < 3 * 256; i += kThreads) lut[i] = lut_g[i];
  for (int i = tid; i < 2 * kFeatPad / 8; i += kThreads)
    reinterpret_cast<uint4*>(tab)[i] = reinterpret_cast<const uint4*>(&g_feat.off[0][0])[i];
#pragma unroll
  for (int k = 0; k < kLoadsPerThread; ++k)
    if (dst[k] >= 0) {
      stage[dst[k]] = v[k].a;
      stage[dst[k] + 1] = v[k].b;
      stage[dst[k] + 2] = v[k].c;
    }
  __syncthreads();

  // q walks the block's output run in memory order: 16-row group, 32-feature block, row,
  // chunk position; the position holds feature chunk kt_chunk(row, position).
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(stage);
  uint16_t* xb = x + u0 * 4 * kFeatPad;   // = first element of the block's first row group
  for (int q = tid; q < kUnitsPerBlock * kChunksPerUnit; q += kThreads) {
    const int grp = q / (kColBlocks * 64), rem0 = q - grp * (kColBlocks * 64);
    const int kb = rem0 >> 6, r16 = (rem0 >> 2) & 15, pos = rem0 & 3;
    const int br = grp * 16 + r16;   // row within the block
    const int u = br >> 2, rr = br & 3;   // unit, row in unit (dh, dw)
    if (u >= nu) continue;
    const int k8 = kb * 4 + kt_chunk(u0 * 4 + br, pos);   // feature chunk
    const int shift = (rr >> 1) * (kPatch * kRowBytes) + (rr & 1) * (kPatch * 3);
    const int kind = sud[u].fstride == 0;   // 1: image (one frame for both slots)
    const uint8_t* ub = sb + u * kUnitBytes + shift;
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    if (k8 < kPadChunk) {   // a chunk lies in one channel; pad chunks stay zero
      const int ch = k8 >= 2 * kChanChunks ? 2 : k8 >= kChanChunks ? 1 : 0;
      const uint4 t4 = *reinterpret_cast<const uint4*>(tab + kind * kFeatPad + 8 * k8);
      const uint32_t tw[4] = {t4.x, t4.y, t4.z, t4.w};
      if constexpr (AFFINE) {
        const float a = ch == 0 ? na.a[0] : ch == 1 ? na.a[1] : na.a[2];
        const float b = ch == 0 ? na.b[0] : ch == 1 ? na.b[1] : na.b[2];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          packed[h] = pack_bf16(__builtin_fmaf((float)ub[tw[h] & 0xffffu], a, b),
                                __builtin_fmaf((float)ub[tw[h] >> 16], a, b));
      } else {
        const uint16_t* L = lut + ch * 256;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          packed[h] = (uint32_t)L[ub[tw[h] & 0xffffu]] | ((uint32_t)L[ub[tw[h] >> 16]] << 16);
      }
    }
    // streaming output: nontemporal stores (the rows are read once, by the next kernel)
    __builtin_nontemporal_store(u32x4{packed[0], packed[1], packed[2], packed[3]},
                                reinterpret_cast<u32x4*>(xb + (int64_t)q * 8));
  }
}

// uint8 flatten_patches rows [N][1176] -> blocked bf16 [N][1184]; 8 features per thread
// (1176 = 147 * 8 and 392 = 49 * 8, so a chunk never straddles a channel).
__global__ void __launch_bounds__(kThreads)
normrows_kernel(const uint8_t* __restrict__ patches, int64_t n_rows,
                const uint16_t* __restrict__ lut_g, uint16_t* __restrict__ x) {
  __shared__ uint16_t lut[3 * 256];
  for (int i = threadIdx.x; i < 3 * 256; i += kThreads) lut[i] = lut_g[i];
  __syncthreads();
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= n_rows * kChunksPerRow) return;
  const int64_t row = j / kChunksPerRow;
  const int k8 = (int)(j % kChunksPerRow);
  uint4 pk = make_uint4(0, 0, 0, 0);
  if (8 * k8 < kFeat) {
    const uint2 raw = *reinterpret_cast<const uint2*>(patches + row * kFeat + 8 * k8);
    const uint16_t* L = lut + (8 * k8 / 392) * 256;
    auto b = [&](uint32_t w, int s) { return (uint32_t)L[(w >> (8 * s)) & 0xff]; };
    pk.x = b(raw.x, 0) | (b(raw.x, 1) << 16);
    pk.y = b(raw.x, 2) | (b(raw.x, 3) << 16);
    pk.z = b(raw.y, 0) | (b(raw.y, 1) << 16);
    pk.w = b(raw.y, 2) | (b(raw.y, 3) << 16);
  }
  *reinterpret_cast<uint4*>(x + kt_index(row, 8 * k8, kFeatPad)) = pk;
}

}  // namespace

vit_status launch_normpatch(const uint8_t* pixels, const UnitDesc* units, int64_t n_units,
                            const uint16_t* lut, const NormAffine* affine, uint16_t* x, void* stream,
                            const int32_t* n_units_dev) {
  if (n_units <= 0) return VIT_OK;
  const int64_t blocks = (n_units + kUnitsPerBlock - 1) / kUnitsPerBlock;
  if (affine)
    hipLaunchKernelGGL(normpatch_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), pixels, units, n_units, n_units_dev, lut, *affine, x);
  else
    hipLaunchKernelGGL(normpatch_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), pixels, units, n_units, n_units_dev, lut, NormAffine{},
                       x);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("normpatch launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

vit_status launch_normrows_u8(const uint8_t* patches, int64_t n_rows, const uint16_t* lut,
                              uint16_t* x, void* stream) {
  if (n_rows <= 0) return VIT_OK;
  const int64_t blocks = (n_rows * kChunksPerRow + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(normrows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), patches, n_rows, lut, x);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("normrows launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

}  // namespace vitmi
