// Row normalisation of the float32 residual stream into bfloat16 GEMM inputs.
//
// LayerNorm (Qwen2-VL tower) or RMSNorm (Qwen2.5-VL tower) over the hidden
// width with eps 1e-6 (vLLM PR #55370 report, key code: the towers take a
// norm epsilon defaulting to 1e-6; "vLLM multimodal inference | ViT
// performance optimisation", section 3.5 names RMSNorm among the fused ops).
// One wave per row; the row stays in registers, so the statistics are exact
// two-pass sums in float32; output is rounded to nearest-even bfloat16 and
// stored in the blocked layout the GEMMs load (kt_index).
#include <hip/hip_runtime.h>

#include "vit_internal.h"

namespace vitmi {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ float bf16_lo(float x) {
  return x - (float)(__bf16)x;
}

// VPL = float4 chunks per lane (d <= 256 * VPL).  SPLIT: each output row is
// [hi | lo] with hi = bf16(y) and lo = bf16(y - hi).  Input row `row` lands in blocked row
// row / group at column offset (row % group) * S * d of a group * S * d wide matrix.
template <int KIND, int VPL, bool SPLIT, bool DYN>
__global__ void __launch_bounds__(kThreads)
rownorm_kernel(const float* __restrict__ r, int64_t rows, const int32_t* __restrict__ rows_dev, int d,
               const float* __restrict__ g, const float* __restrict__ b, float eps, int group,
               uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= (DYN ? (int64_t)*rows_dev : rows)) return;   // DYN: run-time count (bucketed graph)
  const float4* src = reinterpret_cast<const float4*>(r + row * d);
  const int n4 = d >> 2;
  float4 v[VPL];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < n4 ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (KIND == VIT_NORM_LAYER) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  float mean = 0.f;
  if (KIND == VIT_NORM_LAYER) mean = wave_sum(s) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = lane + 64 * i;
    if (c < n4) {
      const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
      q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
  const int w = d * (SPLIT ? 2 : 1);
  const int64_t orow = row / group;
  const int ocol = (int)(row % group) * w, ocols = group * w;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = lane + 64 * i;
    if (c < n4) {
      const float4 gg = g4[c];
      float4 y;
      y.x = (v[i].x - mean) * rstd * gg.x;
      y.y = (v[i].y - mean) * rstd * gg.y;
      y.z = (v[i].z - mean) * rstd * gg.z;
      y.w = (v[i].w - mean) * rstd * gg.w;
      if (KIND == VIT_NORM_LAYER) {
        const float4 bb = b4[c];
        y.x += bb.x; y.y += bb.y; y.z += bb.z; y.w += bb.w;
      }
      *reinterpret_cast<uint2*>(out + kt_index(orow, ocol + 4 * c, ocols)) =
          make_uint2(pack_bf16(y.x, y.y), pack_bf16(y.z, y.w));
      if (SPLIT)
        *reinterpret_cast<uint2*>(out + kt_index(orow, ocol + d + 4 * c, ocols)) =
            make_uint2(pack_bf16(bf16_lo(y.x), bf16_lo(y.y)), pack_bf16(bf16_lo(y.z), bf16_lo(y.w)));
    }
  }
}

// Two rows per wave (rows 2w, 2w + 1 of a 16-row group share each 128-byte line of the blocked
// layout): lanes 0-31 take the even row, lanes 32-63 the odd one, so every store instruction
// writes whole lines.  VPL2 = float4 chunks per lane per row (d <= 128 * VPL2).
template <int KIND, int VPL2, bool SPLIT, bool DYN>
__global__ void __launch_bounds__(kThreads)
rownorm2_kernel(const float* __restrict__ r, int64_t rows, const int32_t* __restrict__ rows_dev, int d,
                const float* __restrict__ g, const float* __restrict__ b, float eps, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, hl = lane >> 5, c32 = lane & 31;
  const int64_t row = ((int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6)) * 2 + hl;
  const int64_t nrows = DYN ? (int64_t)*rows_dev : rows;
  const bool live = row < nrows;
  const float4* src = reinterpret_cast<const float4*>(r + (live ? row : 0) * d);
  const int n4 = d >> 2;
  float4 v[VPL2];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL2; ++i) {
    const int c = c32 + 32 * i;
    v[i] = (live && c < n4) ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (KIND == VIT_NORM_LAYER) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  auto half_sum = [](float x) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
  };
  float mean = 0.f;
  if (KIND == VIT_NORM_LAYER) mean = half_sum(s) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPL2; ++i) {
    const int c = c32 + 32 * i;
    if (c < n4) {
      const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
      q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float rstd = 1.0f / sqrtf(half_sum(q) / (float)d + eps);
  if (!live) return;
  const int w = d * (SPLIT ? 2 : 1);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
  for (int i = 0; i < VPL2; ++i) {
    const int c = c32 + 32 * i;
    if (c < n4) {
      const float4 gg = g4[c];
      float4 y;
      y.x = (v[i].x - mean) * rstd * gg.x;
      y.y = (v[i].y - mean) * rstd * gg.y;
      y.z = (v[i].z - mean) * rstd * gg.z;
      y.w = (v[i].w - mean) * rstd * gg.w;
      if (KIND == VIT_NORM_LAYER) {
        const float4 bb = b4[c];
        y.x += bb.x; y.y += bb.y; y.z += bb.z; y.w += bb.w;
      }
      *reinterpret_cast<uint2*>(out + kt_index(row, 4 * c, w)) =
          make_uint2(pack_bf16(y.x, y.y), pack_bf16(y.z, y.w));
      if (SPLIT)
        *reinterpret_cast<uint2*>(out + kt_index(row, d + 4 * c, w)) =
            make_uint2(pack_bf16(bf16_lo(y.x), bf16_lo(y.y)), pack_bf16(bf16_lo(y.z), bf16_lo(y.w)));
    }
  }
}

template <int KIND, bool SPLIT>
vit_status launch_kind(const float* r, int64_t rows, const int32_t* rows_dev, int d, const float* g,
                       const float* b, float eps, int group, uint16_t* out, hipStream_t st) {
  if (group == 1 && d == 1280) {   // the tower's width: two rows per wave
    const dim3 grid2((unsigned)((rows + 2 * kRowsPerBlock - 1) / (2 * kRowsPerBlock)));
    if (rows_dev)
      hipLaunchKernelGGL((rownorm2_kernel<KIND, 10, SPLIT, true>), grid2, dim3(kThreads), 0, st, r, rows, rows_dev,
                         d, g, b, eps, out);
    else
      hipLaunchKernelGGL((rownorm2_kernel<KIND, 10, SPLIT, false>), grid2, dim3(kThreads), 0, st, r, rows, rows_dev,
                         d, g, b, eps, out);
    return VIT_OK;
  }
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const int vpl = (d / 4 + 63) / 64;
#define VIT_ROWNORM(V)                                                                                  \
  if (rows_dev)                                                                                         \
    hipLaunchKernelGGL((rownorm_kernel<KIND, V, SPLIT, true>), grid, dim3(kThreads), 0, st, r, rows,    \
                       rows_dev, d, g, b, eps, group, out);                                             \
  else                                                                                                  \
    hipLaunchKernelGGL((rownorm_kernel<KIND, V, SPLIT, false>), grid, dim3(kThreads), 0, st, r, rows,   \
                       rows_dev, d, g, b, eps, group, out);
  if (vpl <= 1) {
    VIT_ROWNORM(1)
  } else if (vpl <= 2) {
    VIT_ROWNORM(2)
  } else if (vpl <= 5) {
    VIT_ROWNORM(5)
  } else if (vpl <= 8) {
    VIT_ROWNORM(8)
  } else {
    set_error("rownorm: hidden %d too wide (max 2048)", d);
    return VIT_E_ARG;
  }
#undef VIT_ROWNORM
  return VIT_OK;
}

// Debug copy: blocked bf16 -> row-major, 4 values (one 8-byte piece of a chunk) per thread.
__global__ void __launch_bounds__(kThreads)
unblock_kernel(const uint16_t* __restrict__ src, int64_t rows, int cols, int group, int out_cols,
               uint16_t* __restrict__ dst) {
  const int q4 = out_cols / 4;
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= rows * q4) return;
  const int64_t m = j / q4;
  const int c = (int)(j % q4) * 4;
  const int64_t s = kt_index(m / group, (m % group) * cols + c, (int64_t)group * cols);
  *reinterpret_cast<uint2*>(dst + m * out_cols + c) = *reinterpret_cast<const uint2*>(src + s);
}

}  // namespace

vit_status launch_unblock(const uint16_t* src, int64_t rows, int cols, int group, int out_cols,
                          uint16_t* dst, void* stream) {
  if (rows <= 0) return VIT_OK;
  if (cols % 32 || out_cols % 4 || out_cols > cols || group < 1) {
    set_error("unblock: bad shape cols=%d out_cols=%d group=%d", cols, out_cols, group);
    return VIT_E_ARG;
  }
  const int64_t blocks = (rows * (out_cols / 4) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(unblock_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     src, rows, cols, group, out_cols, dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("unblock launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

vit_status launch_rownorm(int kind, const float* r, int64_t rows, int d, const float* g,
                          const float* b, float eps, uint16_t* out, bool split, int group,
                          void* stream, const int32_t* rows_dev) {
  if (rows <= 0) return VIT_OK;
  if (d % 32 || group < 1 || rows % group) {
    set_error("rownorm: hidden %d must be a multiple of 32 and rows %lld a multiple of the group %d", d,
              (long long)rows, group);
    return VIT_E_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  vit_status s;
  if (kind == VIT_NORM_LAYER)
    s = split ? launch_kind<VIT_NORM_LAYER, true>(r, rows, rows_dev, d, g, b, eps, group, out, st)
              : launch_kind<VIT_NORM_LAYER, false>(r, rows, rows_dev, d, g, b, eps, group, out, st);
  else
    s = split ? launch_kind<VIT_NORM_RMS, true>(r, rows, rows_dev, d, g, b, eps, group, out, st)
              : launch_kind<VIT_NORM_RMS, false>(r, rows, rows_dev, d, g, b, eps, group, out, st);
  if (s != VIT_OK) return s;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("rownorm launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

}  // namespace vitmi
