// normpatch: uint8 HWC frames -> bfloat16 flatten_patches rows, in one pass.
//
// The tower's first step rescales and normalises integer pixels into the
// tower dtype (vLLM PR #55370 report, implementation breakdown); patchify
// cuts 14x14 patches over two temporal slots, keeps each 2x2 merge unit's
// rows adjacent and flattens features in (channel, slot, row, column) order
// ("vLLM multimodal inference | ViT performance optimisation", sections 2.2
// and 3.2).  The normalised value of every (channel, byte) pair is taken from
// a 3x256 table of exactly rounded bfloat16 values, so the result is the
// correctly rounded quotient bit for bit.
//
// One workgroup handles kUnitsPerBlock merge units.  Each unit's 2 slots x 28
// pixel rows x 84 bytes are staged in LDS with dword loads, then every thread
// emits 16-byte chunks of the 4 output rows (1184 bf16 each; columns
// 1176..1183 are zero so the patch-embed GEMM needs no K tail).
#include <hip/hip_runtime.h>

#include "vit_internal.h"

namespace vitmi {

namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerBlock = 4;
constexpr int kRowBytes = kUnitPx * 3;                        // 84
constexpr int kUnitBytes = kTemporal * kUnitPx * kRowBytes;   // 4704
constexpr int kUnitDwords = kUnitBytes / 4;                   // 1176
constexpr int kChunksPerRow = kFeatPad / 8;                   // 148
constexpr int kChunksPerUnit = 4 * kChunksPerRow;             // 608

__global__ void __launch_bounds__(kThreads)
normpatch_kernel(const uint8_t* __restrict__ pixels, const UnitDesc* __restrict__ units,
                 int64_t n_units, const uint16_t* __restrict__ lut_g, uint16_t* __restrict__ x) {
  __shared__ uint32_t stage[kUnitsPerBlock][kUnitDwords];
  __shared__ uint16_t lut[3 * 256];
  const int tid = threadIdx.x;
  for (int i = tid; i < 3 * 256; i += kThreads) lut[i] = lut_g[i];

  const int64_t u0 = (int64_t)blockIdx.x * kUnitsPerBlock;
  const int nu = (int)min<int64_t>(kUnitsPerBlock, n_units - u0);
  // stage: dword j of a unit -> slot = j / (28*21), row = (j / 21) % 28, dword-in-row = j % 21
  for (int j = tid; j < nu * kUnitDwords; j += kThreads) {
    const int u = j / kUnitDwords, jj = j % kUnitDwords;
    const UnitDesc ud = units[u0 + u];
    const int slot = jj / (kUnitPx * 21), rem = jj % (kUnitPx * 21);
    const int row = rem / 21, dw = rem % 21;
    const uint8_t* src = pixels + ud.px_off + (int64_t)slot * ud.fstride + (int64_t)row * ud.pitch + 4 * dw;
    stage[u][jj] = *reinterpret_cast<const uint32_t*>(src);
  }
  __syncthreads();

  for (int j = tid; j < nu * kChunksPerUnit; j += kThreads) {
    const int u = j / kChunksPerUnit, jj = j % kChunksPerUnit;
    const int rr = jj / kChunksPerRow, k8 = jj % kChunksPerRow;   // row in unit (dh, dw), chunk
    const int dh = rr >> 1, dwc = rr & 1;
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(stage[u]);
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int f = 8 * k8 + e;
      if (f < kFeat) {
        const int c = f / 392, r1 = f % 392;
        const int tau = r1 / 196, r2 = r1 % 196;
        const int i = r2 / 14, jx = r2 % 14;
        const int y = kPatch * dh + i, xx = kPatch * dwc + jx;
        v[e] = lut[c * 256 + sb[(tau * kUnitPx + y) * kRowBytes + xx * 3 + c]];
      } else {
        v[e] = 0;
      }
    }
    uint4 pk;
    pk.x = v[0] | ((uint32_t)v[1] << 16);
    pk.y = v[2] | ((uint32_t)v[3] << 16);
    pk.z = v[4] | ((uint32_t)v[5] << 16);
    pk.w = v[6] | ((uint32_t)v[7] << 16);
    const int64_t row = 4 * (u0 + u) + rr;
    *reinterpret_cast<uint4*>(x + row * kFeatPad + 8 * k8) = pk;
  }
}

// uint8 flatten_patches rows [N][1176] -> bf16 [N][1184]; 8 features per thread
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
  *reinterpret_cast<uint4*>(x + row * kFeatPad + 8 * k8) = pk;
}

}  // namespace

vit_status launch_normpatch(const uint8_t* pixels, const UnitDesc* units, int64_t n_units,
                            const uint16_t* lut, uint16_t* x, void* stream) {
  if (n_units <= 0) return VIT_OK;
  const int64_t blocks = (n_units + kUnitsPerBlock - 1) / kUnitsPerBlock;
  hipLaunchKernelGGL(normpatch_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), pixels, units, n_units, lut, x);
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
