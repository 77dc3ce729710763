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
// registers, and each lane owns the running max of the one query its O^T
// columns belong to.  The softmax denominator comes out of the same MFMA
// chain: one extra 16-row tile of O^T multiplies P by an all-ones operand.
// Online softmax in fp32 with exp2 and the 1/sqrt(d) scale folded into the
// exponent; P is rounded to bf16 for the MFMA.  The running max is only
// raised (and O, l rescaled) when a block's max exceeds it by more than 2^8,
// which keeps the rescale off the common path without changing the math.
//
// Per-score VALU work is what bounds this kernel on CDNA4 (exp runs at a
// quarter of the FMA rate), so a step is 32 keys x 64 queries per wave, the
// whole state fits in 256 registers and two waves share each SIMD, letting
// one wave's MFMAs run under the other's softmax.  K tiles (32 keys x head_dim,
// row stride head_dim + 8) and V^T tiles (head_dim x 32 keys, row stride 36)
// move global -> LDS with gfx950's direct loads into a double-buffered ring.
// Work units are laid out so each XCD (workgroups are dispatched round-robin
// over 8 XCDs) runs contiguous (head, segment) ranges and shares their K/V in
// its L2.  Long segments use 4-wave workgroups (256 queries share each K/V
// tile); short segments (windows) use 1-wave workgroups of 64 queries.
#include <hip/hip_runtime.h>

#include <cmath>

#include "vit_internal.h"

namespace vitmi {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int KB = 32;   // keys per step

// max over lanes l and l ^ 16 (rows of 16 lanes swapped pairwise in registers, no LDS trip)
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}
// max over lanes l and l ^ 32
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}
constexpr int QT = 4;    // 16-query tiles per wave (64 queries)

template <int HD, int NW>
__global__ void __launch_bounds__(NW * 64, 2)
attn_kernel(AttnArgs a, const AttnWork* __restrict__ work, int n_work) {
  constexpr int KS = HD + 8;             // K tile row stride (elements): 16-byte chunks
  constexpr int KCH = KS / 8;            // chunks per LDS row (the last one is padding)
  constexpr int KLOADS = (KB * KCH + 63) / 64;     // 1 KB direct loads per K tile
  constexpr int VS = KB + 4;             // V^T tile row stride (elements)
  constexpr int VDW = VS / 2;            // dwords per V^T row
  constexpr int VLOADS = (HD * VDW + 63) / 64;     // 256 B direct loads per V^T tile
  // 32-wide reduction chunks of the head dim; with head_dim = 16 (mod 32) the last chunk
  // holds 16 dims in its first two lane groups and zeros in the other two (a 16x16x16 MFMA
  // costs as many cycles as a 16x16x32 one, so the padding is free)
  constexpr int NC = (HD + 31) / 32;
  constexpr bool TAIL = (HD % 32) == 16;
  constexpr int ND = HD / 16;
  static_assert(HD % 16 == 0 && (KS * 2) % 16 == 0, "head_dim must be a multiple of 16");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][KLOADS * 64 * 8];
  __shared__ __attribute__((aligned(16))) uint32_t sV[2][VLOADS * 64];

  // ---- work unit: XCD-contiguous ranges of (head, unit), units of a segment adjacent
  const int G = n_work * a.heads;
  const int pid = blockIdx.x;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + local;
  const int head = logical / n_work;
  const AttnWork wk = work[logical % n_work];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int seg0 = wk.seg_start, n = wk.seg_len;
  const int qbase = wk.q0 + wv * 64;
  const uint16_t* Qh = a.q + (int64_t)head * a.n_tok * HD;
  const uint16_t* Kh = a.k + (int64_t)head * a.n_tok * HD;
  const uint16_t* Vh = a.vt + (int64_t)head * HD * a.n_tok;

  // ---- this wave's query fragments (B operand of S^T = K Q^T)
  bf16x8 qa[QT][NC];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int q = qbase + 16 * t + l16;
    const bool ok = q < n;
    const uint16_t* qr = Qh + (int64_t)(seg0 + (ok ? q : 0)) * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bool live = ok && (!TAIL || c < NC - 1 || g4 < 2);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + (live ? c * 32 + g4 * 8 : 0));
      qa[t][c] = live ? v : bf16x8{};
    }
  }
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;

  f32x4 O[ND][QT], Ls[QT];   // O^T tiles and the row-sum tile (every row holds l)
  float m[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m[t] = 0.f;
    Ls[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) O[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc = 1.4426950408889634f / sqrtf((float)HD);   // log2(e) / sqrt(head_dim)
  const int nkb = (n + KB - 1) / KB;

  // Direct global -> LDS tile loads.  Keys past the segment end read the last key (K) or
  // the last key pair (V^T): their scores are masked to -inf, so they contribute P = 0.
  auto dload = [&](int kb, int buf) {
    const int key0 = kb * KB;
#pragma unroll
    for (int j = 0; j < (KLOADS + NW - 1) / NW; ++j) {
      const int i = wv + j * NW;
      if (i >= KLOADS) break;
      const int id = i * 64 + lane, r = id / KCH, c = id % KCH;
      const int key = min(key0 + r, n - 1);
      const uint16_t* src = Kh + (int64_t)(seg0 + key) * HD + (c < HD / 8 ? c * 8 : 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(&sK[buf][i * 64 * 8]), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < (VLOADS + NW - 1) / NW; ++j) {
      const int i = wv + j * NW;
      if (i >= VLOADS) break;
      const int id = i * 64 + lane, dd = id / VDW, c = id % VDW;
      const int key = min(key0 + 2 * c, n - 2);
      const uint16_t* src = (dd < HD && c < KB / 2) ? Vh + (int64_t)dd * a.n_tok + seg0 + key : Vh;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(&sV[buf][i * 64]), 4, 0, 0);
    }
  };

  dload(0, 0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) dload(kb + 1, buf ^ 1);
    if (qbase < n) {
      const uint16_t* Kt = sK[buf];
      const uint16_t* Vt = reinterpret_cast<const uint16_t*>(sV[buf]);
      // ---- S^T tiles: 2 key tiles x QT query tiles
      f32x4 S[2][QT];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint16_t* kr = Kt + (kt * 16 + l16) * KS;
        bf16x8 ka[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[c] = *reinterpret_cast<const bf16x8*>(kr + c * 32 + g4 * 8);
        // upper lane groups of a half chunk read the row padding and the next row: zero them
        if constexpr (TAIL) ka[NC - 1] = g4 < 2 ? ka[NC - 1] : bf16x8{};
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          f32x4 s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qa[t][c], s, 0, 0, 0);
          S[kt][t] = s;
        }
      }
      // ---- mask keys past the segment end (last step only)
      const int key_base = kb * KB;
      if (key_base + KB > n) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key_base + kt * 16 + g4 * 4 + i >= n)
#pragma unroll
              for (int t = 0; t < QT; ++t) S[kt][t][i] = -INFINITY;
      }
      // ---- online softmax per query column (lazy offset: raised only by > 2^8)
      bf16x8 pb[QT];
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        float mx = fmaxf(fmaxf(fmaxf(S[0][t][0], S[0][t][1]), fmaxf(S[0][t][2], S[0][t][3])),
                         fmaxf(fmaxf(S[1][t][0], S[1][t][1]), fmaxf(S[1][t][2], S[1][t][3])));
        mx = max_xor32(max_xor16(mx));
        const float bm = mx * sc;
        if (kb == 0) {
          m[t] = bm;
        } else {
          const bool need = bm > m[t] + 8.0f;
          if (__builtin_amdgcn_ballot_w64(need)) {
            const float mn = need ? bm : m[t];
            const float alpha = __builtin_amdgcn_exp2f(m[t] - mn);
            m[t] = mn;
            Ls[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) O[dt][t] *= alpha;
          }
        }
        const float mo = m[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[t][i] = (__bf16)__builtin_amdgcn_exp2f(S[0][t][i] * sc - mo);
          pb[t][4 + i] = (__bf16)__builtin_amdgcn_exp2f(S[1][t][i] * sc - mo);
        }
      }
      // ---- O^T += V^T P^T (and l += 1^T P^T) over the 32 keys
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const uint16_t* vr = Vt + (dt * 16 + l16) * VS + g4 * 4;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int t = 0; t < QT; ++t) O[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[t], O[dt][t], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < QT; ++t) Ls[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[t], Ls[t], 0, 0, 0);
    }
    __syncthreads();
  }

  if (qbase >= n) return;
  const int ld = a.heads * HD;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int q = qbase + 16 * t + l16;
    if (q < n) {
      const float inv = 1.0f / Ls[t][0];
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
    hipLaunchKernelGGL((attn_kernel<HD, 4>), dim3(a.n_long * a.heads), dim3(256), 0, st, a, a.work_long,
                       a.n_long);
  if (a.n_short > 0)
    hipLaunchKernelGGL((attn_kernel<HD, 1>), dim3(a.n_short * a.heads), dim3(64), 0, st, a, a.work_short,
                       a.n_short);
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
