// Content keys of the items' uint8 pixels, for the vision-embedding cache (reuse merged
// embeddings across requests keyed by the pixels and the grid: "vLLM multimodal inference |
// ViT performance optimisation", section 2.3).
//
// Key of an item whose pixel bytes form L/8 little-endian 64-bit words w_0, w_1, ...:
//   lane j in {0, 1}:  S_j = sum_i mix(w_i + (i + 1) * G_j)  (mod 2^64)
//   key_j = mix(S_j ^ (L * G_j))
// with G_0 = 0x9e3779b97f4a7c15, G_1 = 0xd1b54a32d192ed03 and mix() the 64-bit finaliser of
// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
// OOPSLA 2014; shifts 30, 27, 31 with the multipliers below).  The sum makes the key
// independent of the order in which workgroups add their partial sums, so it is exact and
// deterministic; the word index inside each term makes it position-dependent.  A 128-bit
// content key, not a cryptographic one.  The kernel computes S_j; the host applies the
// final mix.
#include <hip/hip_runtime.h>

#include "vit_internal.h"

namespace vitmi {

namespace {

constexpr int kThreads = 256;
constexpr int kWordsPerThread = 32;                        // 16 x 16-byte loads
constexpr int64_t kWordsPerBlock = (int64_t)kThreads * kWordsPerThread;   // 64 KB of pixels

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
  return ((uint64_t)hi << 32) | lo;
}

// grid: x = 64 KB chunk of an item, y = item.  items[i] = {byte offset, word count}.
__global__ void __launch_bounds__(kThreads)
pixel_hash_kernel(const uint8_t* __restrict__ pixels, const int64_t* __restrict__ items,
                  unsigned long long* __restrict__ sums) {
  const int item = blockIdx.y;
  const int64_t off = items[2 * item], words = items[2 * item + 1];
  const int64_t w0 = (int64_t)blockIdx.x * kWordsPerBlock;
  if (w0 >= words) return;
  const uint64_t* src = reinterpret_cast<const uint64_t*>(pixels + off);
  uint64_t s0 = 0, s1 = 0;
#pragma unroll 4
  for (int k = 0; k < kWordsPerThread / 2; ++k) {
    // pairs of consecutive words per 16-byte load; consecutive threads take consecutive pairs
    const int64_t i = w0 + 2 * ((int64_t)k * kThreads + threadIdx.x);
    if (i >= words) break;
    const uint4 v = *reinterpret_cast<const uint4*>(src + i);
    const uint64_t a = ((uint64_t)v.y << 32) | v.x, b = ((uint64_t)v.w << 32) | v.z;
    const uint64_t n = (uint64_t)i + 1;
    s0 += mix64(a + n * 0x9e3779b97f4a7c15ull) + mix64(b + (n + 1) * 0x9e3779b97f4a7c15ull);
    s1 += mix64(a + n * 0xd1b54a32d192ed03ull) + mix64(b + (n + 1) * 0xd1b54a32d192ed03ull);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    s0 += shfl_xor64(s0, o);
    s1 += shfl_xor64(s1, o);
  }
  __shared__ uint64_t part[2][kThreads / 64];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    part[0][wv] = s0;
    part[1][wv] = s1;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    uint64_t t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t += part[threadIdx.x][w];
    atomicAdd(sums + 2 * item + threadIdx.x, (unsigned long long)t);
  }
}

__global__ void zero_u64_kernel(unsigned long long* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

vit_status launch_pixel_hash(const uint8_t* pixels, const int64_t* items_dev, int n_items, int64_t max_words,
                             uint64_t* sums_dev, void* stream) {
  if (n_items <= 0) return VIT_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_u64_kernel, dim3((2 * n_items + 255) / 256), dim3(256), 0, st,
                     reinterpret_cast<unsigned long long*>(sums_dev), 2 * n_items);
  const int64_t chunks = (max_words + kWordsPerBlock - 1) / kWordsPerBlock;
  if (chunks > 0)
    hipLaunchKernelGGL(pixel_hash_kernel, dim3((unsigned)chunks, (unsigned)n_items), dim3(kThreads), 0, st,
                       pixels, items_dev, reinterpret_cast<unsigned long long*>(sums_dev));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("pixel hash launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

}  // namespace vitmi
