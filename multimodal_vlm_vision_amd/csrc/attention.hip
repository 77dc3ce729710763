// Block-diagonal (varlen) flash attention for the vision tower on gfx950.
//
// For every segment s and head h: O_s = softmax(Q_s K_s^T / sqrt(head_dim)) V_s,
// with segments = items (cu_seqlens; attention never crosses an image
// boundary: "vLLM multimodal inference | ViT performance optimisation",
// section 3.4) or, in window-attention layers, windows laid out contiguously
// by the planner (section 3.3).  A tile never spans two segments: every work
// unit names its segment and the kernel only reads that segment's keys.
//
// Formulation: the wave computes S^T = K Q^T (keys as MFMA rows, queries as
// columns) with v_mfma_f32_16x16x32_bf16 (+16x16x16 for a 16-wide head_dim
// tail), so each lane ends up holding 4 consecutive keys of one query.  Those
// probabilities are already the B operand of O^T = V^T P^T (the 32-key
// reduction slots of a lane are its 4 keys of each of two 16-key tiles; V^T
// fragments are read with the same key permutation), so P never leaves
// registers, and each lane owns the running max / sum of the one query its
// O^T columns belong to.  Online softmax in fp32 with exp2 and the 1/sqrt(d)
// scale folded into the exponent; P is rounded to bf16 for the MFMA.
//
// K tiles (64 keys x head_dim, row stride head_dim + 8 elements) and V^T
// tiles (head_dim x 64 keys, row stride 68) are staged in a double-buffered
// LDS ring.  Long segments use 4-wave workgroups (256 queries share each
// K/V tile, next tile prefetched into registers); short segments (windows)
// use 1-wave workgroups of 64 queries.
#include <hip/hip_runtime.h>

#include <cmath>

#include "vit_internal.h"

namespace vitmi {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int KB = 64;   // keys per step
constexpr int QT = 4;    // 16-query tiles per wave (64 queries)

template <int HD, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_kernel(AttnArgs a, const AttnWork* __restrict__ work) {
  constexpr int KS = HD + 8;
  constexpr int VS = KB + 4;
  constexpr int NC = HD / 32;
  constexpr bool TAIL = (HD % 32) == 16;
  constexpr int ND = HD / 16;
  constexpr int NT = NW * 64;
  constexpr int KCH = KB * HD / 8;   // 16-byte chunks per K tile
  constexpr int VCH = HD * KB / 4;   // 8-byte chunks per V^T tile
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VPT = (VCH + NT - 1) / NT;
  static_assert(HD % 16 == 0, "head_dim must be a multiple of 16");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][KB * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][HD * VS];

  const AttnWork wk = work[blockIdx.x];
  const int head = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int seg0 = wk.seg_start, n = wk.seg_len;
  const int qbase = wk.q0 + wv * 64;
  const uint16_t* Qh = a.q + (int64_t)head * a.n_tok * HD;
  const uint16_t* Kh = a.k + (int64_t)head * a.n_tok * HD;
  const uint16_t* Vh = a.vt + (int64_t)head * HD * a.n_tok;

  // ---- this wave's query fragments (B operand of S^T = K Q^T)
  bf16x8 qa[QT][NC];
  bf16x4 qt4[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int q = qbase + 16 * t + l16;
    const bool ok = q < n;
    const uint16_t* qr = Qh + (int64_t)(seg0 + (ok ? q : 0)) * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + c * 32 + g4 * 8);
      qa[t][c] = ok ? v : bf16x8{};
    }
    if constexpr (TAIL) {
      bf16x4 v = *reinterpret_cast<const bf16x4*>(qr + NC * 32 + g4 * 4);
      qt4[t] = ok ? v : bf16x4{};
    }
  }

  f32x4 O[ND][QT];
  float m[QT], l[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) O[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc = 1.4426950408889634f / sqrtf((float)HD);   // log2(e) / sqrt(head_dim)
  const int nkb = (n + KB - 1) / KB;

  uint4 rk[KPT];
  uint2 rv[VPT];
  auto gload = [&](int kb) {
    const int key0 = kb * KB;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int id = tid + i * NT;
      if (id < KCH) {
        const int r = id / (HD / 8), c = id % (HD / 8), key = key0 + r;
        rk[i] = key < n ? *reinterpret_cast<const uint4*>(Kh + (int64_t)(seg0 + key) * HD + c * 8)
                        : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int id = tid + i * NT;
      if (id < VCH) {
        const int dd = id / (KB / 4), c = id % (KB / 4), key = key0 + 4 * c;
        rv[i] = key < n ? *reinterpret_cast<const uint2*>(Vh + (int64_t)dd * a.n_tok + seg0 + key)
                        : make_uint2(0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int id = tid + i * NT;
      if (id < KCH) {
        const int r = id / (HD / 8), c = id % (HD / 8);
        *reinterpret_cast<uint4*>(&sK[buf][r * KS + c * 8]) = rk[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int id = tid + i * NT;
      if (id < VCH) {
        const int dd = id / (KB / 4), c = id % (KB / 4);
        *reinterpret_cast<uint2*>(&sV[buf][dd * VS + 4 * c]) = rv[i];
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (NW > 1 && kb + 1 < nkb) gload(kb + 1);
    if (qbase < n) {
      // ---- S^T tiles: 4 key tiles x QT query tiles
      f32x4 S[4][QT];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint16_t* kr = &sK[buf][(kt * 16 + l16) * KS];
        bf16x8 ka[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[c] = *reinterpret_cast<const bf16x8*>(kr + c * 32 + g4 * 8);
        bf16x4 kb4{};
        if constexpr (TAIL) kb4 = *reinterpret_cast<const bf16x4*>(kr + NC * 32 + g4 * 4);
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          f32x4 s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qa[t][c], s, 0, 0, 0);
          if constexpr (TAIL) s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kb4, qt4[t], s, 0, 0, 0);
          S[kt][t] = s;
        }
      }
      // ---- mask keys past the segment end (last step only)
      const int key_base = kb * KB;
      if (key_base + KB > n) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key_base + kt * 16 + g4 * 4 + i >= n)
#pragma unroll
              for (int t = 0; t < QT; ++t) S[kt][t][i] = -INFINITY;
      }
      // ---- online softmax per query column
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        float mx = S[0][t][0];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kt][t][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m[t], mx * sc);
        const float alpha = __builtin_amdgcn_exp2f(m[t] - mnew);
        m[t] = mnew;
        float ls = l[t] * alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) O[dt][t] *= alpha;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(S[kt][t][i] * sc - mnew);
            S[kt][t][i] = pv;
            ls += pv;
          }
        l[t] = ls;
      }
      // ---- O^T += V^T P^T over two 32-key chunks
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 pb[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pb[t][i] = (__bf16)S[2 * j][t][i];
            pb[t][4 + i] = (__bf16)S[2 * j + 1][t][i];
          }
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const uint16_t* vr = &sV[buf][(dt * 16 + l16) * VS + 32 * j + g4 * 4];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
          const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int t = 0; t < QT; ++t) O[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[t], O[dt][t], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkb) {
      if (NW == 1) gload(kb + 1);
      sstore((kb + 1) & 1);
    }
    __syncthreads();
  }

  if (qbase >= n) return;
  const int ld = a.heads * HD;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float ls = l[t];
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    const int q = qbase + 16 * t + l16;
    if (q < n) {
      const float inv = 1.0f / ls;
      uint16_t* orow = a.o + (int64_t)(seg0 + q) * ld + head * HD + g4 * 4;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        uint2 pk;
        pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(O[dt][t][0] * inv)) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(O[dt][t][1] * inv)) << 16);
        pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(O[dt][t][2] * inv)) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(O[dt][t][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + dt * 16) = pk;
      }
    }
  }
}

template <int HD>
hipError_t run_hd(const AttnArgs& a, hipStream_t st) {
  if (a.n_long > 0)
    hipLaunchKernelGGL((attn_kernel<HD, 4>), dim3(a.n_long, a.heads), dim3(256), 0, st, a, a.work_long);
  if (a.n_short > 0)
    hipLaunchKernelGGL((attn_kernel<HD, 1>), dim3(a.n_short, a.heads), dim3(64), 0, st, a, a.work_short);
  return hipGetLastError();
}

}  // namespace

vit_status launch_attention(const AttnArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (a.head_dim) {
    case 32: e = run_hd<32>(a, st); break;
    case 64: e = run_hd<64>(a, st); break;
    case 80: e = run_hd<80>(a, st); break;
    default:
      set_error("attention: head_dim %d not supported (32, 64, 80)", a.head_dim);
      return VIT_E_ARG;
  }
  if (e != hipSuccess) {
    set_error("attention launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

}  // namespace vitmi
