// Device resize of decoded uint8 images to the tower's 28-pixel grid, before the path
// ("vLLM multimodal inference | ViT performance optimisation", section 2.2: the preprocessor
// resizes, pads and normalises images into pixel tensors; SGLang PR #35349 report: CPU
// preprocessing caps request throughput).  The pages fix neither the target size nor the
// interpolation; the readings here:
//   * each side goes to the nearest multiple of 28 pixels (half up), at least 28;
//   * bilinear sampling with half-pixel centres (source coordinate (d + 0.5) * S / D - 0.5,
//     clamped to the image), no antialiasing, channels and frames independent;
//   * weights in 11-bit fixed point and integer arithmetic throughout, output rounded half
//     up, so the result is exact and identical on any implementation of the same rule.
// Frames are HWC RGB uint8, row-major, `frames` of them back to back (source and output).
#include <hip/hip_runtime.h>

#include "vit_internal.h"

namespace vitmi {

namespace {

constexpr int kThreads = 256;
constexpr int kQ = 11;               // fixed-point weight bits
constexpr int kOne = 1 << kQ;

// Source index and weight of the second neighbour for output coordinate d of D, source S:
// s = ((2d + 1) S - D) / (2D), i0 = floor(s) clamped, w = round((s - i0) * 2^11).  32-bit
// arithmetic: sides are at most 8192, so (2d + 1) S < 2^31.
__device__ __forceinline__ void axis(int d, int D, int S, int& i0, int& i1, int& w) {
  const int num = (2 * d + 1) * S - D;   // s * 2D
  const int den = 2 * D;
  if (num <= 0) {
    i0 = 0; i1 = 0; w = 0;
    return;
  }
  const int q = (int)((unsigned)num / (unsigned)den);
  const int r = num - q * den;
  if (q >= S - 1) {
    i0 = S - 1; i1 = S - 1; w = 0;
    return;
  }
  i0 = q;
  i1 = q + 1;
  w = (int)(((unsigned)r * kOne + (unsigned)(den / 2)) / (unsigned)den);   // in [0, 2^11]
}

// Rows of source bytes a workgroup of R output rows reads: output rows y .. y + R - 1 sample
// source rows floor(s(y)) .. floor(s(y + R - 1)) + 1, and S / D <= 41 / 28 for every side the
// resize rule produces, so (3 R) / 2 + 3 rows always suffice.
__host__ __device__ constexpr int src_rows_for(int R) { return (3 * R) / 2 + 3; }

// One workgroup per R consecutive output rows of one frame: the source rows they read are
// staged in LDS (dword loads from each row's dword-aligned start; bytes past the buffer read as
// zero and are never used) together with a per-column table (x0 | wx << 16; the second
// neighbour is x0 + 1 when wx > 0), then each thread produces whole output dwords (an output
// row is dw * 3 bytes, a multiple of 4 since dw is a multiple of 28).  src and dst are 4-byte
// aligned.
__global__ void __launch_bounds__(kThreads)
resize_rows_kernel(const uint8_t* __restrict__ src, int sh, int sw, uint8_t* __restrict__ dst, int dh, int dw,
                   uint32_t src_bytes, int R) {
  extern __shared__ uint32_t lds[];
  const int blocks_per_frame = (dh + R - 1) / R;
  const int f = blockIdx.x / blocks_per_frame;
  const int ys = (blockIdx.x - f * blocks_per_frame) * R;
  const int nr = min(R, dh - ys);
  int ya, yb, w_unused;
  axis(ys, dh, sh, ya, yb, w_unused);
  int yc, yd;
  axis(ys + nr - 1, dh, sh, yc, yd, w_unused);
  const int srow0 = ya, nsrc = yd - ya + 1;           // <= src_rows_for(R)
  const int rb = sw * 3;                               // bytes per source row
  const int nd = rb / 4 + 2;                           // dwords covering a row from its aligned start
  uint32_t* xtab = lds;                                // dw entries
  uint32_t* rows = lds + dw;                           // nsrc rows of nd dwords
  for (int x = threadIdx.x; x < dw; x += kThreads) {
    int x0, x1, wx;
    axis(x, dw, sw, x0, x1, wx);
    xtab[x] = (uint32_t)x0 | ((uint32_t)wx << 16);
  }
  const uint32_t base = (uint32_t)(f * sh + srow0) * (uint32_t)rb;
  for (int i = threadIdx.x; i < nsrc * nd; i += kThreads) {
    const int r = i / nd, k = i - r * nd;
    const uint32_t a = ((base + (uint32_t)r * rb) & ~3u) + 4u * (uint32_t)k;
    uint32_t v = 0;
    if (a + 4 <= src_bytes) {
      v = *reinterpret_cast<const uint32_t*>(src + a);
    } else {   // the buffer's last, partial dword (or past the end: never used)
      for (uint32_t q = 0; q < 4; ++q)
        if (a + q < src_bytes) v |= (uint32_t)src[a + q] << (8 * q);
    }
    rows[i] = v;
  }
  __syncthreads();
  const int nw = dw * 3 / 4;
  for (int yy = 0; yy < nr; ++yy) {
    const int y = ys + yy;
    int y0, y1, wy;
    axis(y, dh, sh, y0, y1, wy);
    const uint8_t* L0 = reinterpret_cast<const uint8_t*>(rows + (y0 - srow0) * nd) +
                        ((base + (uint32_t)(y0 - srow0) * rb) & 3u);
    const uint8_t* L1 = reinterpret_cast<const uint8_t*>(rows + (y1 - srow0) * nd) +
                        ((base + (uint32_t)(y1 - srow0) * rb) & 3u);
    uint32_t* out = reinterpret_cast<uint32_t*>(dst + ((size_t)f * dh + y) * dw * 3);
    for (int j = threadIdx.x; j < nw; j += kThreads) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int byte = 4 * j + b, p = byte / 3, c = byte - 3 * p;
        const uint32_t t = xtab[p];
        const int x0 = (int)(t & 0xffffu), wx = (int)(t >> 16), x1 = wx ? x0 + 1 : x0;
        const int top = (kOne - wx) * L0[3 * x0 + c] + wx * L0[3 * x1 + c];
        const int bot = (kOne - wx) * L1[3 * x0 + c] + wx * L1[3 * x1 + c];
        const int v = ((kOne - wy) * top + wy * bot + (1 << (2 * kQ - 1))) >> (2 * kQ);
        word |= (uint32_t)v << (8 * b);
      }
      out[j] = word;
    }
  }
}

}  // namespace

int resize_side(int s) {
  const int m = (s + 14) / 28;   // nearest multiple of 28, half up
  return 28 * (m < 1 ? 1 : m);
}

vit_status launch_resize(const uint8_t* src, int sh, int sw, int frames, uint8_t* dst, int dh, int dw,
                         void* stream) {
  if ((int64_t)dh * frames <= 0) return VIT_OK;
  const int64_t src_bytes = (int64_t)frames * sh * sw * 3;
  const size_t row = (size_t)(sw * 3 / 4 + 2) * 4, tab = (size_t)dw * 4;
  const size_t budget = 160 * 1024;
  if (sh > 8192 || sw > 8192 || src_bytes >= ((int64_t)1 << 32) || tab + src_rows_for(1) * row > budget) {
    set_error("resize: image too large (sides <= 8192 px, source < 4 GiB)");
    return VIT_E_SHAPE;
  }
  // one output row per workgroup: measured fastest (time grew linearly with the rows per
  // workgroup, 1 -> 8 on 48 images of ~1344^2: 0.65 -> 1.66 ms; the per-row loop is the bound)
  const int R = 1;
  const size_t lds = tab + src_rows_for(R) * row;
  const int64_t blocks = (int64_t)frames * ((dh + R - 1) / R);
  if (blocks >= ((int64_t)1 << 31)) {
    set_error("resize: too many output rows");
    return VIT_E_SHAPE;
  }
  if (lds > 64 * 1024) {   // wide rows: raise the dynamic LDS limit (current device)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(resize_rows_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
      set_error("resize LDS attribute: %s", hipGetErrorString(e));
      return VIT_E_HIP;
    }
  }
  hipLaunchKernelGGL(resize_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), lds,
                     static_cast<hipStream_t>(stream), src, sh, sw, dst, dh, dw, (uint32_t)src_bytes, R);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("resize launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

}  // namespace vitmi
