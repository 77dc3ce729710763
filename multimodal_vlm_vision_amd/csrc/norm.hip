// Row normalisation of the float32 residual stream into 16-bit GEMM inputs.
//
// LayerNorm (Qwen2-VL tower) or RMSNorm (Qwen2.5-VL tower) over the hidden
// width with eps 1e-6 (vLLM PR #55370 report, key code: the towers take a
// norm epsilon defaulting to 1e-6; "vLLM multimodal inference | ViT
// performance optimisation", section 3.5 names RMSNorm among the fused ops).
// One wave per row (two rows per wave at the tower's width 1280, so every store
// writes whole lines); the row stays in registers, so the statistics are exact
// two-pass sums in float32; output is rounded to nearest-even float16 (the default
// activation form) or bfloat16 and stored in the blocked layout the GEMMs load
// (kt_index), with the compensated bf16 forms' second part (a bfloat16 lo half,
// or an e4m3 residual in kt8_index).
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

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// two floats -> packed float16 pair, round to nearest even (one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// AM 3 (float16 activations): float16 pairs; otherwise bfloat16 pairs
template <int AM>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (AM == 3) return pack_f16(a, b);
  else return pack_bf16(a, b);
}

__device__ __forceinline__ float bf16_lo(float x) {
  return x - (float)(__bf16)x;
}

// residual x - bf16(x) times 2^kLoShift, clamped to e4m3's finite range, for four values -> four
// OCP e4m3 bytes (round to nearest even)
__device__ __forceinline__ uint32_t lo_e4m3x4(float4 y) {
  constexpr float s = (float)(1 << kLoShift);
  auto f = [](float x) { return fminf(fmaxf(bf16_lo(x) * s, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f(y.x), f(y.y), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f(y.z), f(y.w), lo, true);
}

// VPL = float4 chunks per lane (d <= 256 * VPL).  AM 0: bf16 rows; AM 1: each output row is
// [hi | lo] with hi = bf16(y) and lo = bf16(y - hi); AM 2: hi rows, and the e4m3 residuals
// (times 2^kLoShift) at the same place of out8 (kt8_index); AM 3: float16 rows.  Input row `row` lands in blocked row
// row / group at column offset (row % group) * S * d of a group * S * d wide matrix.
template <int KIND, int VPL, int AM, bool DYN>
__global__ void __launch_bounds__(kThreads)
rownorm_kernel(const float* __restrict__ r, int64_t rows, const int32_t* __restrict__ rows_dev, int d,
               const float* __restrict__ g, const float* __restrict__ b, float eps, int group,
               uint16_t* __restrict__ out, uint8_t* __restrict__ out8) {
  constexpr bool SPLIT = AM == 1;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= (DYN ? (int64_t)*rows_dev : rows)) return;   // DYN: run-time count (bucketed graph)
  const float4* src = reinterpret_cast<const float4*>(r + row * d);
  const int n4 = d >> 2;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
  // the row, its gains and shifts all read before the first store
  float4 v[VPL], gv[VPL], bv[VPL];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < n4 ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    gv[i] = c < n4 ? g4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    bv[i] = (KIND == VIT_NORM_LAYER && c < n4) ? b4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
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
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = lane + 64 * i;
    if (c < n4) {
      const float4 gg = gv[i];
      float4 y;
      y.x = (v[i].x - mean) * rstd * gg.x;
      y.y = (v[i].y - mean) * rstd * gg.y;
      y.z = (v[i].z - mean) * rstd * gg.z;
      y.w = (v[i].w - mean) * rstd * gg.w;
      if (KIND == VIT_NORM_LAYER) {
        const float4 bb = bv[i];
        y.x += bb.x; y.y += bb.y; y.z += bb.z; y.w += bb.w;
      }
      *reinterpret_cast<uint2*>(out + kt_index(orow, ocol + 4 * c, ocols)) =
          make_uint2(pack16<AM>(y.x, y.y), pack16<AM>(y.z, y.w));
      if (SPLIT)
        *reinterpret_cast<uint2*>(out + kt_index(orow, ocol + d + 4 * c, ocols)) =
            make_uint2(pack_bf16(bf16_lo(y.x), bf16_lo(y.y)), pack_bf16(bf16_lo(y.z), bf16_lo(y.w)));
      if (AM == 2) *reinterpret_cast<uint32_t*>(out8 + kt8_index(orow, ocol + 4 * c, ocols)) = lo_e4m3x4(y);
    }
  }
}

// Two rows per wave (rows 2w, 2w + 1 of a 16-row group share each 128-byte line of the blocked
// layout): lanes 0-31 take the even row, lanes 32-63 the odd one, so every store instruction
// writes whole lines.  VPL2 = float4 chunks per lane per row (d <= 128 * VPL2).
template <int KIND, int VPL2, int AM, bool DYN>
__global__ void __launch_bounds__(kThreads)
rownorm2_kernel(const float* __restrict__ r, int64_t rows, const int32_t* __restrict__ rows_dev, int d,
                const float* __restrict__ g, const float* __restrict__ b, float eps, uint16_t* __restrict__ out,
                uint8_t* __restrict__ out8) {
  constexpr bool SPLIT = AM == 1;
  const int lane = threadIdx.x & 63, hl = lane >> 5, c32 = lane & 31;
  const int64_t row = ((int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6)) * 2 + hl;
  const int64_t nrows = DYN ? (int64_t)*rows_dev : rows;
  const bool live = row < nrows;
  const float4* src = reinterpret_cast<const float4*>(r + (live ? row : 0) * d);
  const int n4 = d >> 2;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
  // the row, its gains and shifts all read before the first store (a read after a store would
  // wait for it: the compiler cannot tell the output from the inputs)
  float4 v[VPL2], gv[VPL2], bv[VPL2];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL2; ++i) {
    const int c = c32 + 32 * i;
    v[i] = (live && c < n4) ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    gv[i] = c < n4 ? g4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    bv[i] = (KIND == VIT_NORM_LAYER && c < n4) ? b4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
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
#pragma unroll
  for (int i = 0; i < VPL2; ++i) {
    const int c = c32 + 32 * i;
    if (c < n4) {
      const float4 gg = gv[i];
      float4 y;
      y.x = (v[i].x - mean) * rstd * gg.x;
      y.y = (v[i].y - mean) * rstd * gg.y;
      y.z = (v[i].z - mean) * rstd * gg.z;
      y.w = (v[i].w - mean) * rstd * gg.w;
      if (KIND == VIT_NORM_LAYER) {
        const float4 bb = bv[i];
        y.x += bb.x; y.y += bb.y; y.z += bb.z; y.w += bb.w;
      }
      *reinterpret_cast<uint2*>(out + kt_index(row, 4 * c, w)) =
          make_uint2(pack16<AM>(y.x, y.y), pack16<AM>(y.z, y.w));
      if (SPLIT)
        *reinterpret_cast<uint2*>(out + kt_index(row, d + 4 * c, w)) =
            make_uint2(pack_bf16(bf16_lo(y.x), bf16_lo(y.y)), pack_bf16(bf16_lo(y.z), bf16_lo(y.w)));
      if (AM == 2) *reinterpret_cast<uint32_t*>(out8 + kt8_index(row, 4 * c, d)) = lo_e4m3x4(y);
    }
  }
}

template <int KIND, int AM>
vit_status launch_kind(const float* r, int64_t rows, const int32_t* rows_dev, int d, const float* g,
                       const float* b, float eps, int group, uint16_t* out, uint8_t* out8, hipStream_t st) {
  if (group == 1 && d == 1280) {   // the tower's width: two rows per wave
    const dim3 grid2((unsigned)((rows + 2 * kRowsPerBlock - 1) / (2 * kRowsPerBlock)));
    if (rows_dev)
      hipLaunchKernelGGL((rownorm2_kernel<KIND, 10, AM, true>), grid2, dim3(kThreads), 0, st, r, rows, rows_dev,
                         d, g, b, eps, out, out8);
    else
      hipLaunchKernelGGL((rownorm2_kernel<KIND, 10, AM, false>), grid2, dim3(kThreads), 0, st, r, rows, rows_dev,
                         d, g, b, eps, out, out8);
    return VIT_OK;
  }
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const int vpl = (d / 4 + 63) / 64;
#define VIT_ROWNORM(V)                                                                                  \
  if (rows_dev)                                                                                         \
    hipLaunchKernelGGL((rownorm_kernel<KIND, V, AM, true>), grid, dim3(kThreads), 0, st, r, rows,       \
                       rows_dev, d, g, b, eps, group, out, out8);                                       \
  else                                                                                                  \
    hipLaunchKernelGGL((rownorm_kernel<KIND, V, AM, false>), grid, dim3(kThreads), 0, st, r, rows,      \
                       rows_dev, d, g, b, eps, group, out, out8);
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

// Debug copy of a bf16 + e4m3-residual activation: row m -> [hi(out_cols) | residual(out_cols)]
// as bf16, the residual decoded (v_cvt_f32_fp8) and scaled back by 2^-kLoShift (exact in bf16).
__global__ void __launch_bounds__(kThreads)
unblock_f8_kernel(const uint16_t* __restrict__ src, const uint8_t* __restrict__ src8, int64_t rows, int cols,
                  int group, int out_cols, uint16_t* __restrict__ dst) {
  const int q4 = out_cols / 4;
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= rows * q4) return;
  const int64_t m = j / q4;
  const int c = (int)(j % q4) * 4;
  const int64_t ld = (int64_t)group * cols, rr = m / group, cc = (m % group) * cols + c;
  uint16_t* o = dst + m * 2 * out_cols;
  *reinterpret_cast<uint2*>(o + c) = *reinterpret_cast<const uint2*>(src + kt_index(rr, cc, ld));
  const int v = *reinterpret_cast<const int*>(src8 + kt8_index(rr, cc, ld));
  constexpr float s = 1.0f / (float)(1 << kLoShift);
  *reinterpret_cast<uint2*>(o + out_cols + c) =
      make_uint2(pack_bf16(__builtin_amdgcn_cvt_f32_fp8(v, 0) * s, __builtin_amdgcn_cvt_f32_fp8(v, 1) * s),
                 pack_bf16(__builtin_amdgcn_cvt_f32_fp8(v, 2) * s, __builtin_amdgcn_cvt_f32_fp8(v, 3) * s));
}

}  // namespace

vit_status launch_unblock_f8(const uint16_t* src, const uint8_t* src8, int64_t rows, int cols, int group,
                             int out_cols, uint16_t* dst, void* stream) {
  if (rows <= 0) return VIT_OK;
  if (cols % 32 || out_cols % 4 || out_cols > cols || group < 1) {
    set_error("unblock_f8: bad shape cols=%d out_cols=%d group=%d", cols, out_cols, group);
    return VIT_E_ARG;
  }
  const int64_t blocks = (rows * (out_cols / 4) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(unblock_f8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), src, src8, rows, cols, group, out_cols, dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("unblock_f8 launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

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
                          void* stream, const int32_t* rows_dev, uint8_t* out8, bool f16) {
  if (rows <= 0) return VIT_OK;
  if (d % 32 || group < 1 || rows % group || ((int)split + (out8 != nullptr) + (int)f16 > 1)) {
    set_error("rownorm: hidden %d must be a multiple of 32 and rows %lld a multiple of the group %d "
              "(and at most one of split / out8 / f16)", d, (long long)rows, group);
    return VIT_E_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int am = f16 ? 3 : out8 ? 2 : split ? 1 : 0;
  vit_status s;
#define VIT_NORM_AM(K)                                                                   \
  (am == 3   ? launch_kind<K, 3>(r, rows, rows_dev, d, g, b, eps, group, out, out8, st) \
   : am == 2 ? launch_kind<K, 2>(r, rows, rows_dev, d, g, b, eps, group, out, out8, st) \
   : am == 1 ? launch_kind<K, 1>(r, rows, rows_dev, d, g, b, eps, group, out, out8, st) \
             : launch_kind<K, 0>(r, rows, rows_dev, d, g, b, eps, group, out, out8, st))
  s = kind == VIT_NORM_LAYER ? VIT_NORM_AM(VIT_NORM_LAYER) : VIT_NORM_AM(VIT_NORM_RMS);
#undef VIT_NORM_AM
  if (s != VIT_OK) return s;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("rownorm launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

}  // namespace vitmi
