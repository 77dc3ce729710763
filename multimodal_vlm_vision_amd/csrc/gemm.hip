// bf16 MFMA GEMM for gfx950 with fused epilogues.
//
// C[M][N] = A[M][K] * B[N][K]^T: both operands in the blocked layout of
// kt_index (16 rows x 32 K per 1 KB block; activations [tokens][features],
// weights [out][in]), fp32 accumulation in v_mfma_f32_32x32x16_bf16.  Used for every dense product of the tower:
// patch embedding (the stride = kernel 3D conv as one GEMM, "vLLM multimodal
// inference | ViT performance optimisation", section 3.2), qkv, out-proj,
// MLP and the merger MLP (sections 2.2 and 3.1).  The small elementwise steps
// that follow a product are fused into its epilogue (section 3.5): bias,
// exact-erf GELU, SiLU(gate)*up, residual add into the fp32 stream, the 2D
// RoPE of q and k (section 3.3), and the merger's row scatter.
//
// Split activations: an A row may hold each activation as a pair
// hi = bf16(x), lo = bf16(x - hi), laid out in groups of g columns
// ([hi(g) | lo(g)] repeated).  The kernel then accumulates hi*w + lo*w
// against ONE copy of the weight tile: every B fragment read from LDS feeds
// two MFMAs, so the pair costs twice the MFMA work but not twice the B
// traffic.
//
// bf16 + e4m3 residual activations (A8 set): the same compensation with the
// residual x - bf16(x) stored as OCP e4m3 (times 2^9, one byte) in a separate
// fp8 matrix, multiplied against an e4m3 copy of the weights whose rows carry
// power-of-two E8M0 scales.  gfx950's scaled fp8 MFMA (32x32x64, per-row A and
// per-column B scales) adds that product into the same fp32 accumulators and
// undoes both scales on the way, at ~0.43 of the MFMA time of a second bf16
// product; the residual's own error (e4m3's 3 mantissa bits on a term ~2^-9 of
// x) stays ~2^-12 of x.  The fp8 MFMA takes 64 K per instruction: with a
// 32-column stage, each stage's 32 residual bytes of a row fill half of the
// operand (lanes 0-31 the first 16 bytes of both stages, lanes 32-63 the
// second: A and B use the same mapping, so the products still pair equal k).
//
// Main loop (per workgroup tile BM x BN, 2x2 waves of (BM/2) x (BN/2)):
//  * K advances 32 columns per stage.  Tiles move global -> LDS with gfx950's
//    buffer loads into LDS (no VGPR staging): one 64-lane 16-byte load moves
//    one 1 KB operand block (whole cache lines: rows of 64-byte K slices would
//    touch twice as many lines and halve the CU's load rate); the block's
//    wave-uniform offset and the K advance ride in the scalar offset, the
//    lane's 16 bytes in one vector offset shared by every load.  LDS rows are
//    64 bytes; the blocked layout already puts the four 16-byte chunks of row
//    r at chunk ^ ((r >> 3) & 3), which keeps the 32x32x16 fragment reads
//    (32 rows, one chunk) free of bank conflicts.
//  * A ring of 2-4 stages: a stage's slot is refilled as soon as every wave
//    has read it (the barrier in the middle of the next stage), so each load
//    has S-1 whole stages to land; one barrier per stage, preceded by an
//    exact vmcnt wait for the next stage only.
//  * MFMA operand fragments are double-buffered in registers: the reads for
//    the next 16-wide K step are interleaved with the current step's MFMAs.
//  * Workgroups are remapped so each XCD (dispatch is round-robin over 8
//    XCDs) runs a contiguous range of tiles, grouped group_m row-tiles deep
//    (column tiles vary fastest within a group), to keep A and B panels in
//    its L2.
//
// Epilogue: the accumulators are staged through LDS one 32-row slice at a
// time, so every global access of the epilogue is a 16-byte (fp32) or 8-byte
// (bf16) vector: residual read-modify-write, bias, activations, RoPE pairs
// and the transposed V store all run on 4 consecutive columns (or rows).  A
// slice issues all its global reads before its first store.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "vit_internal.h"

namespace vitmi {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int BK = 32;             // logical K per stage: LDS rows of 64 bytes
constexpr int CPR = BK / 8;        // 16-byte chunks per LDS row
constexpr int RPL = 64 / CPR;      // LDS rows filled by one 64-lane 16-byte load
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit dword format, no swizzle
constexpr int kLdsBytes = 160 * 1024;


// s_waitcnt vmcnt(n) with lgkm and exp counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ uint2 pack4(float4 v) { return make_uint2(pack2(v.x, v.y), pack2(v.z, v.w)); }

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// activation pairs in the operand type of activation mode AM: float16 for AM 3 (one
// v_cvt_pk_f16_f32, round to nearest even), bfloat16 otherwise
template <int AM>
__device__ __forceinline__ uint32_t pack2a(float a, float b) {
  if constexpr (AM == 3) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  else return pack2(a, b);
}
template <int AM>
__device__ __forceinline__ uint2 pack4a(float4 v) {
  return make_uint2(pack2a<AM>(v.x, v.y), pack2a<AM>(v.z, v.w));
}

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26
// (|error| <= 1.5e-7, far below the bf16 rounding of the GELU output).
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly = ((((1.061405429f * t - 1.453152027f) * t + 1.421413741f) * t - 0.284496736f) * t +
                      0.254829592f) * t;
  const float y = 1.0f - poly * __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
  return copysignf(y, x);
}

// exact (erf-form) GELU: x * Phi(x)
__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752f)); }

__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// four floats -> four OCP e4m3 bytes, round to nearest even (two v_cvt_pk_fp8_f32)
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// residual y - hi (exact in fp32) times 2^kLoShift, clamped to e4m3's finite range
__device__ __forceinline__ float lo_scaled(float y, float hi) {
  return fminf(fmaxf((y - hi) * (float)(1 << kLoShift), -448.0f), 448.0f);
}

// bf16 activation store into the blocked layout (ldo columns): hi = bf16(y) of the 8 columns
// n..n+7 (one 16-byte chunk, n % 8 == 0); with split_off, lo = bf16(y - hi) at n + split_off;
// AM 2: the e4m3 residual of the 8 columns (8 bytes) into out8.
template <int AM>
__device__ __forceinline__ void store_act8(const GemmArgs& p, int m, int n, const float (&y)[8]) {
  uint16_t* o = static_cast<uint16_t*>(p.out);
  uint32_t hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hi[i] = pack2a<AM>(y[2 * i], y[2 * i + 1]);
  *reinterpret_cast<uint4*>(o + kt_index(m, n, p.ldo)) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  if constexpr (AM == 3) {
    return;   // float16 activations carry no second part
  } else if constexpr (AM == 2) {
    uint32_t l8[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      l8[i] = pack_e4m3x4(lo_scaled(y[4 * i], __builtin_bit_cast(float, hi[2 * i] << 16)),
                          lo_scaled(y[4 * i + 1], __builtin_bit_cast(float, hi[2 * i] & 0xffff0000u)),
                          lo_scaled(y[4 * i + 2], __builtin_bit_cast(float, hi[2 * i + 1] << 16)),
                          lo_scaled(y[4 * i + 3], __builtin_bit_cast(float, hi[2 * i + 1] & 0xffff0000u)));
    *reinterpret_cast<uint2*>(p.out8 + kt8_index(m, n, p.ldo8)) = make_uint2(l8[0], l8[1]);
  } else if (p.split_off) {
    uint32_t lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lo[i] = pack2(y[2 * i] - __builtin_bit_cast(float, hi[i] << 16),
                    y[2 * i + 1] - __builtin_bit_cast(float, hi[i] & 0xffff0000u));
    *reinterpret_cast<uint4*>(o + kt_index(m, n + p.split_off, p.ldo)) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

// AM (activation mode): 0 single bf16, 1 hi+lo bf16 pairs, 2 bf16 + e4m3 residual, 3 float16
// activations against float16 weights (loaded exactly like mode 0, multiplied on the f16 MFMA)
template <int BM, int BN, int WM, int WN, int AM, int OCC = 1>
struct Geo {
  static constexpr bool SPLIT = AM == 1, F8 = AM == 2;
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int AR = SPLIT ? 2 * BM : BM;        // A rows per stage: hi rows, then lo rows
  static constexpr int ROWS = AR + BN;
  static constexpr int kF8Off = ROWS * BK * 2;           // AM 2: e4m3 A8 then B8 rows (32 B) follow
  static constexpr int NA8 = BM / 32, NB8 = BN / 32;     // AM 2: 1 KB e4m3 blocks per stage
  static constexpr int kStageBytes = kF8Off + (F8 ? (BM + BN) * 32 : 0);
  static constexpr int kStage = kStageBytes / 2;         // bf16 elements per stage
  static constexpr int LA = AR / RPL / NW;               // A loads per wave per stage
  static constexpr int LB = BN / RPL / NW;               // B loads per wave per stage
  // AM 2: e4m3 block loads per wave (a block count that does not split evenly over the waves
  // is rounded up; the extra loads repeat the last block into its own slot)
  static constexpr int LA8 = F8 ? (NA8 + NW - 1) / NW : 0;
  static constexpr int LB8 = F8 ? (NB8 + NW - 1) / NW : 0;
  static constexpr int LPW = LA + LB + LA8 + LB8;
  static constexpr int kBudget = kLdsBytes / OCC;          // OCC workgroups share a CU's LDS
  static constexpr int kFit = kBudget / kStageBytes;
  static constexpr int STAGES = kFit >= 4 ? 4 : kFit;
  static constexpr int SST = TN * 32 + 8;                // epilogue slice row stride (floats)
  static constexpr int kSliceBytes = NW * 32 * SST * 4;  // one fp32 slice per wave
  static constexpr int kRing = STAGES * kStageBytes;
  static constexpr int kSmem = kRing > kSliceBytes ? kRing : kSliceBytes;
  static_assert(TM >= 1 && TN >= 2 && TN % 2 == 0, "wave tile must hold column pairs");
  static_assert(AR % (RPL * NW) == 0 && BN % (RPL * NW) == 0, "load split");
  static_assert(kFit >= 2, "two stages must fit in LDS");
  static_assert(kSmem <= kBudget, "LDS budget");
  static_assert(kStageBytes % 16 == 0 && LA8 <= 4 && LB8 <= 4, "e4m3 stage layout");
  static_assert((STAGES - 1) * LPW < 64, "vmcnt range");
};

// Applies the epilogue to one staged 32-row slice (rows m_base.., columns n_base.., width W = TN*32).
// Every global read of a slice (bias, residual rows, scatter rows, rotary tables) is issued
// before its first store: the compiler cannot tell the outputs from the inputs, so a read
// placed after a store would wait for that store to complete (one memory round trip per
// 16-byte piece instead of one or two per slice).
template <int EPI, int W, int AM>
__device__ __forceinline__ void epilogue_slice(const GemmArgs& p, int M, const float* sc, int m_base, int n_base,
                                               int lane) {
  constexpr int SST = W + 8;
  constexpr int C4 = W / 4;   // float4 chunks per row
  if (EPI == EPI_F32 || EPI == EPI_RES || EPI == EPI_OUT) {
    constexpr int NQ = 32 * C4 / 64;
    static_assert(64 % C4 == 0, "a lane keeps its columns through the slice");
    const int c4 = lane % C4, n = n_base + 4 * c4;
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (EPI != EPI_F32) b = *reinterpret_cast<const float4*>(p.bias + n);
    float4 res[NQ];
    int orow[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int m = m_base + (lane + 64 * q) / C4;
      if (EPI == EPI_RES)
        res[q] = m < M ? *reinterpret_cast<const float4*>(static_cast<const float*>(p.out) + (int64_t)m * p.ldo + n)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      if (EPI == EPI_OUT) orow[q] = m < M ? p.row_map[m] : 0;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int r = (lane + 64 * q) / C4, m = m_base + r;
      if (m >= M) continue;
      const float4 v = *reinterpret_cast<const float4*>(sc + r * SST + 4 * c4);
      float* o = static_cast<float*>(p.out);
      if (EPI == EPI_F32)
        *reinterpret_cast<float4*>(o + (int64_t)m * p.ldo + n) = v;
      else if (EPI == EPI_RES)
        *reinterpret_cast<float4*>(o + (int64_t)m * p.ldo + n) = f4add(res[q], f4add(v, b));
      else
        *reinterpret_cast<float4*>(o + (int64_t)orow[q] * p.ldo + n) = f4add(v, b);
    }
  } else if (EPI == EPI_GELU || EPI == EPI_SWIGLU) {
    // bf16 activations into the blocked layout: a lane produces one 16-byte chunk (8 columns)
    // of hi (and one of lo), so the 64 lanes of a store write one whole 1 KB block.  The lane's
    // chunk position in the block is q; it holds logical chunk kt_chunk(row, q).
    constexpr int OW = EPI == EPI_SWIGLU ? W / 2 : W;   // output columns of the slice
    constexpr int OB = OW / 32;                          // output column blocks
    constexpr int NB = 2 * OB;                           // (row group, column block) pairs
    const int r16 = lane >> 2, q = lane & 3;
    // GELU: bias of the 8 columns; SwiGLU: bias of the 8 gate and the 8 up columns
    float4 bg[NB][2], bu[NB][2];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int rg = blk / OB, ob = blk % OB;
      const int c = kt_chunk(m_base + 16 * rg + r16, q);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (EPI == EPI_GELU) {
          bg[blk][h] = *reinterpret_cast<const float4*>(p.bias + n_base + 32 * ob + 8 * c + 4 * h);
        } else {
          bg[blk][h] = *reinterpret_cast<const float4*>(p.bias + n_base + 64 * ob + 8 * c + 4 * h);
          bu[blk][h] = *reinterpret_cast<const float4*>(p.bias + n_base + 64 * ob + 8 * c + 32 + 4 * h);
        }
      }
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int rg = blk / OB, ob = blk % OB;
      const int r = 16 * rg + r16, m = m_base + r;
      if (m >= M) continue;
      const int c = kt_chunk(m, q);
      float y[8];
      int oc;
      if (EPI == EPI_GELU) {
        const int cl = 32 * ob + 8 * c;
        oc = n_base + cl;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 x = f4add(*reinterpret_cast<const float4*>(sc + r * SST + cl + 4 * h), bg[blk][h]);
          y[4 * h] = gelu(x.x); y[4 * h + 1] = gelu(x.y); y[4 * h + 2] = gelu(x.z); y[4 * h + 3] = gelu(x.w);
        }
      } else {
        // gate columns cl.., up columns cl + 32.. of the slice's 64-column block ob
        const int cl = 64 * ob + 8 * c;
        oc = n_base / 2 + 32 * ob + 8 * c;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 g = f4add(*reinterpret_cast<const float4*>(sc + r * SST + cl + 4 * h), bg[blk][h]);
          const float4 u = f4add(*reinterpret_cast<const float4*>(sc + r * SST + cl + 32 + 4 * h), bu[blk][h]);
          y[4 * h] = silu(g.x) * u.x; y[4 * h + 1] = silu(g.y) * u.y;
          y[4 * h + 2] = silu(g.z) * u.z; y[4 * h + 3] = silu(g.w) * u.w;
        }
      }
      store_act8<AM>(p, m, oc, y);
    }
  } else if (EPI == EPI_QKV && n_base < 2 * p.hidden) {
    // q is stored times q_scale (the attention kernel's log2(e) / sqrt(head_dim)), applied
    // before the bf16 rounding.
    // pairs: columns c (c % 64 < 32) and c + 32 of each 64-column block.  A lane rotates 8
    // consecutive rotary pairs of one head (head_dim/2 is a multiple of 8 and the frequency
    // count per axis, head_dim/4, a multiple of 4, so each group of 4 has one axis) and writes
    // each member half as one 16-byte store.  The lane's columns are the same in every row.
    constexpr int G8 = W / 16;   // first-member groups of 8 per row
    constexpr int NQ = 32 * G8 / 64;
    static_assert(64 % G8 == 0, "a lane keeps its columns through the slice");
    const int d = p.hidden, hd = p.head_dim, rr = hd / 2, nf = p.nfreq;
    const int g = lane % G8;
    const int cl = (g / 4) * 64 + (g % 4) * 8;          // local column of the first member
    const int n = n_base + cl;
    const int part = n / d, jj = n - part * d;
    const int pair = 32 * (jj / 64) + (jj % 64);
    const int head = pair / rr, kk = pair % rr;
    const float qs = part == 0 ? p.q_scale : 1.0f;
    float4 ba[2], bb[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      ba[hf] = *reinterpret_cast<const float4*>(p.bias + n + 4 * hf);
      bb[hf] = *reinterpret_cast<const float4*>(p.bias + n + 32 + 4 * hf);
    }
    int pos[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int m = m_base + (lane + 64 * q) / G8;
      pos[q] = m < M ? p.row_pos[m] : 0;
    }
    float4 cs[NQ][2], sn[NQ][2];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int k4 = kk + 4 * hf;
        const int ax = k4 < nf ? (pos[q] >> 16) : (pos[q] & 0xffff);
        const int fi = k4 < nf ? k4 : k4 - nf;
        cs[q][hf] = *reinterpret_cast<const float4*>(p.cos_tab + ax * nf + fi);
        sn[q][hf] = *reinterpret_cast<const float4*>(p.sin_tab + ax * nf + fi);
      }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int r = (lane + 64 * q) / G8, m = m_base + r;
      if (m >= M) continue;
      uint32_t w1[4], w2[4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float4 a = f4add(*reinterpret_cast<const float4*>(sc + r * SST + cl + 4 * hf), ba[hf]);
        const float4 b = f4add(*reinterpret_cast<const float4*>(sc + r * SST + cl + 32 + 4 * hf), bb[hf]);
        const float4 c = cs[q][hf], s = sn[q][hf];
        const uint2 u1 = pack4a<AM>(make_float4((a.x * c.x - b.x * s.x) * qs, (a.y * c.y - b.y * s.y) * qs,
                                                (a.z * c.z - b.z * s.z) * qs, (a.w * c.w - b.w * s.w) * qs));
        const uint2 u2 = pack4a<AM>(make_float4((b.x * c.x + a.x * s.x) * qs, (b.y * c.y + a.y * s.y) * qs,
                                                (b.z * c.z + a.z * s.z) * qs, (b.w * c.w + a.w * s.w) * qs));
        w1[2 * hf] = u1.x; w1[2 * hf + 1] = u1.y;
        w2[2 * hf] = u2.x; w2[2 * hf + 1] = u2.y;
      }
      uint16_t* o = (part == 0 ? p.q : p.k) + ((int64_t)head * p.n_tok + m) * hd;
      *reinterpret_cast<uint4*>(o + kk) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
      *reinterpret_cast<uint4*>(o + kk + rr) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
    }
  } else if (EPI == EPI_QKV) {
    // V part: transposed store [head][dim][token]; an item is 8 consecutive rows of one column,
    // one 16-byte store (the V^T pitch is a multiple of 8).  A last group with only 4 valid
    // rows (row counts are multiples of 4) stores those 4: the pad columns must stay zero.
    constexpr int NQ = 4 * W / 64;
    const int d = p.hidden, hd = p.head_dim;
    float bv[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) bv[q] = p.bias[n_base + (lane + 64 * q) / 4];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int id = lane + 64 * q, rg = id % 4, c = id / 4;
      const int m = m_base + 8 * rg, n = n_base + c;
      if (m >= M) continue;
      const float b = bv[q];
      const float4 v0 = make_float4(sc[(8 * rg + 0) * SST + c] + b, sc[(8 * rg + 1) * SST + c] + b,
                                    sc[(8 * rg + 2) * SST + c] + b, sc[(8 * rg + 3) * SST + c] + b);
      const float4 v1 = make_float4(sc[(8 * rg + 4) * SST + c] + b, sc[(8 * rg + 5) * SST + c] + b,
                                    sc[(8 * rg + 6) * SST + c] + b, sc[(8 * rg + 7) * SST + c] + b);
      const int nn = n - 2 * d, head = nn / hd, dd = nn % hd;
      uint16_t* o = p.vt + ((int64_t)head * hd + dd) * p.vt_ld + m;
      const uint2 u0 = pack4a<AM>(v0);
      if (m + 8 <= M) {
        const uint2 u1 = pack4a<AM>(v1);
        *reinterpret_cast<uint4*>(o) = make_uint4(u0.x, u0.y, u1.x, u1.y);
      } else {
        *reinterpret_cast<uint2*>(o) = u0;
      }
    }
  }
}

// DYN: M comes from device memory at run time (bucketed graphs); a separate instantiation, so
// the plain path keeps M as a launch constant.
template <int BM, int BN, int WM, int WN, int AM, int EPI, int OCC, bool DYN>
__global__ void __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
gemm_kernel(GemmArgs p) {
  using G = Geo<BM, BN, WM, WN, AM, OCC>;
  constexpr bool SPLIT = G::SPLIT, F8 = G::F8;
  constexpr int TM = G::TM, TN = G::TN, LA = G::LA, LB = G::LB, S = G::STAGES, AR = G::AR;
  constexpr int LA8 = G::LA8, LB8 = G::LB8;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv % WM, wn = wv / WM;

  // ---- tile index: XCD-contiguous ranges, then grouped row-major order
  // M at run time when a bucketed graph passes it in device memory (the grid covers the
  // capacity; workgroups past this batch's tiles leave at once)
  const int M = DYN ? *p.m_dev : p.M;
  const int gm = (M + BM - 1) / BM, gn = (p.N + BN - 1) / BN;
  const int Gt = gm * gn;
  const int pid = blockIdx.x;
  if (pid >= Gt) return;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = Gt >> 3, rem = Gt & 7;
  const int logical = xcd * per + min(xcd, rem) + local;
  const int in_group = p.group_m * gn;
  const int grp = logical / in_group, first_m = grp * p.group_m;
  const int gsz = min(gm - first_m, p.group_m);
  const int li = logical % in_group;
  const int m0 = (first_m + li % gsz) * BM, n0 = (li / gsz) * BN;

  // ---- load plan: wave wv's j-th load fills stage rows [(wv*LA + j)*16, +16) of A (B likewise)
  // with one operand block; lane l lands at byte 16*l of those rows, where the block keeps it.
  // Row groups past M / N read the last group; those results are never stored.
  static_assert(RPL == 16, "one load = one 16-row block");
  const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.A), (short)0, (int)p.a_bytes,
                                                    kRsrcWord3);
  const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.B), (short)0, (int)p.b_bytes,
                                                    kRsrcWord3);
  // (fixed-size arrays: a dependent bound here fails the host-side instantiation of the split
  // variants with this clang; only the first LA / LB entries are used).  A load's offset is
  // the wave-uniform byte offset of its block (scalar offset, with the K advance) plus the
  // lane's 16 bytes (one vector offset shared by every load).
  static_assert(LA <= 16 && LB <= 16, "load plan");
  uint32_t offa[16], offb[16];
  const uint32_t lane16 = (uint32_t)lane * 16;
  const int last_ga = (M + 15) / 16 - 1, last_gb = p.N / 16 - 1;
  const int64_t kba = p.lda / BK, kbb = p.ldb / BK;   // blocks per row group
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int r = (wv * LA + j) * RPL;   // hi rows [0, BM), then lo rows [BM, 2BM)
    const int g = min((m0 + r % BM) / 16, last_ga);
    offa[j] = (uint32_t)((g * kba + (r >= BM ? p.a_group / BK : 0)) * 1024);
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int g = min((n0 + (wv * LB + j) * RPL) / 16, last_gb);
    offb[j] = (uint32_t)(g * kbb * 1024);
  }
  // AM 2: e4m3 blocks of 32 rows; wave wv's j-th load takes block min(wv * L + j, last) of
  // the stage (A8 then B8), rows past M read the last 32-row group
  uint32_t offa8[4], offb8[4], ldsa8[4], ldsb8[4];
  if constexpr (F8) {
    const int last_g8 = (M + 31) / 32 - 1;
#pragma unroll
    for (int j = 0; j < LA8; ++j) {
      const int b = min(wv * LA8 + j, G::NA8 - 1);
      offa8[j] = (uint32_t)(min((m0 + 32 * b) / 32, last_g8) * (p.lda8 / 32) * 1024);
      ldsa8[j] = (uint32_t)(G::kF8Off + b * 1024);
    }
#pragma unroll
    for (int j = 0; j < LB8; ++j) {
      const int b = min(wv * LB8 + j, G::NB8 - 1);
      offb8[j] = (uint32_t)(((n0 + 32 * b) / 32) * (p.ldb8 / 32) * 1024);
      ldsb8[j] = (uint32_t)(G::kF8Off + (G::NA8 + b) * 1024);
    }
  }
  const auto ra8 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(F8 ? p.A8 : nullptr), (short)0,
                                                     (int)p.a8_bytes, kRsrcWord3);
  const auto rb8 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(F8 ? p.B8 : nullptr), (short)0,
                                                     (int)p.b8_bytes, kRsrcWord3);
  const int nk = p.K / BK;
  auto issue = [&](int kt, int buf) {
    kt = min(kt, nk - 1);   // past the end: reload the last stage into a free slot (never read)
    const int k0 = kt * BK;
    // K block k0 / 32 sits 1 KB after block 0 of its row group (A: hi block; lo is a_group later)
    const uint32_t ka = (uint32_t)((SPLIT ? (k0 / p.a_group) * 2 * p.a_group + k0 % p.a_group : k0) / BK) * 1024;
    const uint32_t kb = (uint32_t)(k0 / BK) * 1024;
    uint16_t* st = smem + buf * G::kStage;
#pragma unroll
    for (int j = 0; j < LA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(st + (wv * LA + j) * RPL * BK), 16, lane16, offa[j] + ka, 0, 0);
#pragma unroll
    for (int j = 0; j < LB; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(st + (AR + (wv * LB + j) * RPL) * BK), 16, lane16,
          offb[j] + kb, 0, 0);
    if constexpr (F8) {
      // K block kt of a 32-row group: 1 KB after block kt - 1
      const uint32_t k8 = (uint32_t)kt * 1024;
      uint8_t* st8 = reinterpret_cast<uint8_t*>(smem) + buf * G::kStageBytes;
#pragma unroll
      for (int j = 0; j < LA8; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra8, (__attribute__((address_space(3))) void*)(st8 + ldsa8[j]), 16,
                                                 lane16, offa8[j] + k8, 0, 0);
#pragma unroll
      for (int j = 0; j < LB8; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb8, (__attribute__((address_space(3))) void*)(st8 + ldsb8[j]), 16,
                                                 lane16, offb8[j] + k8, 0, 0);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment reads: 32x32x16 operand = 32 rows x 16 K; lane -> row lane & 31, chunk 2*kk + lane/32.
  // Fragment rows start at multiples of 32, so a row's chunk permutation (its bits 1-4) is
  // that of lane & 31: one lane offset per kk, the fragment's row base a constant.
  bf16x8 fa[2][TM], fl[2][TM], fb[2][TN];
  const int rl = lane & 31;
  const int lofs[2] = {rl * BK + kt_chunk(rl, lane >> 5) * 8, rl * BK + kt_chunk(rl, 2 + (lane >> 5)) * 8};
  auto lfrag = [&](int buf, int kk, bf16x8 (&xa)[TM], bf16x8 (&xl)[TM], bf16x8 (&xb)[TN]) {
    const uint16_t* st = smem + buf * G::kStage + lofs[kk];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      xa[i] = *reinterpret_cast<const bf16x8*>(st + (wm * TM * 32 + i * 32) * BK);
      if constexpr (SPLIT) xl[i] = *reinterpret_cast<const bf16x8*>(st + (BM + wm * TM * 32 + i * 32) * BK);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) xb[j] = *reinterpret_cast<const bf16x8*>(st + (AR + wn * TN * 32 + j * 32) * BK);
  };
  auto mfma_step = [&](const bf16x8 (&xa)[TM], const bf16x8 (&xl)[TM], const bf16x8 (&xb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (AM == 3)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, xa[i]),
                                                             __builtin_bit_cast(f16x8, xb[j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], xb[j], acc[i][j], 0, 0, 0);
      }
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl[i], xb[j], acc[i][j], 0, 0, 0);
    }
  };
  constexpr int NMF = TM * TN * (SPLIT ? 2 : 1);   // MFMAs per 16-wide K step
  constexpr int NDS = TM * (SPLIT ? 2 : 1) + TN;    // fragment reads per K step

  // Products whose epilogue carries VALU work (GELU, SwiGLU, RoPE) run their main loop at raised
  // wave priority and the epilogue at the normal one, so a co-resident workgroup's epilogue
  // yields issue slots to this one's matrix work (the residual products, whose epilogue is
  // mostly memory traffic, measured no better with it).
  constexpr bool kPrio = EPI == EPI_GELU || EPI == EPI_SWIGLU || EPI == EPI_QKV;
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
  // ---- prologue: every stage in flight, stage 0 landed everywhere
#pragma unroll
  for (int s = 0; s < S; ++s) issue(s, s);
  wait_vm<(S - 1) * G::LPW>();
  __builtin_amdgcn_s_barrier();
  lfrag(0, 0, fa[0], fl[0], fb[0]);

  if constexpr (F8) {
    // e4m3 operand halves: h[0] from an even stage, h[1] from the following odd one.  A stage's
    // half is read right after the barrier that makes it visible (step 1 of the stage before),
    // and the pair's fp8 MFMAs run in step 0 of the odd stage.
    i32x4 ha[2][TM], hb[2][TN];
    // lane -> row lane & 31 of a 32-row block, chunk lane / 32 (swapped when row bit 3 is set)
    const int lofs8 = rl * 32 + ((((lane >> 5) ^ (rl >> 3)) & 1) << 4);
    auto lfrag8 = [&](int buf, i32x4 (&xa)[TM], i32x4 (&xb)[TN]) {
      const uint8_t* s8 = reinterpret_cast<const uint8_t*>(smem) + buf * G::kStageBytes + G::kF8Off + lofs8;
#pragma unroll
      for (int i = 0; i < TM; ++i) xa[i] = *reinterpret_cast<const i32x4*>(s8 + (wm * TM + i) * 1024);
#pragma unroll
      for (int j = 0; j < TN; ++j) xb[j] = *reinterpret_cast<const i32x4*>(s8 + (G::NA8 + wn * TN + j) * 1024);
    };
    // E8M0 scales: A rows 2^-kLoShift, B column n (this lane's column of tile j) 2^(s[n] - 127)
    constexpr int kScaleA = 127 - kLoShift;
    int sb[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = p.b8_scale[n0 + wn * TN * 32 + j * 32 + (lane & 31)];
    auto mfma8 = [&]() {
      i32x8 bv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bv[j] = __builtin_shufflevector(hb[0][j], hb[1][j], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const i32x8 av = __builtin_shufflevector(ha[0][i], ha[1][i], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv[j], acc[i][j], 0, 0, 0, kScaleA, 0,
                                                                     sb[j]);
      }
    };
    constexpr int NMF1 = TM * TN;                // bf16 MFMAs of step 1
    constexpr int NDS1 = 2 * (TM + TN);          // step 1 reads: bf16 and e4m3 fragments
    lfrag8(0, ha[0], hb[0]);
    auto stage = [&](int kt, auto hc) {
      constexpr int h = decltype(hc)::value;
      const int buf = kt % S;
      lfrag(buf, 1, fa[1], fl[1], fb[1]);
      mfma_step(fa[0], fl[0], fb[0]);
      if constexpr (h == 1) mfma8();
#pragma unroll
      for (int i = 0; i < NDS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMF * (h + 1), 0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<(S - 2) * G::LPW>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      lfrag((kt + 1) % S, 0, fa[0], fl[0], fb[0]);
      lfrag8((kt + 1) % S, ha[1 - h], hb[1 - h]);
      issue(kt + S, buf);
      mfma_step(fa[1], fl[1], fb[1]);
#pragma unroll
      for (int i = 0; i < (NDS1 + 1) / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < (G::LPW + 1) / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMF1, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < nk; kt += 2) {
      stage(kt, std::integral_constant<int, 0>{});
      stage(kt + 1, std::integral_constant<int, 1>{});
    }
  } else {
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % S;
    // step 0: MFMAs on K columns [0,16) of stage kt while reading columns [16,32)
    lfrag(buf, 1, fa[1], fl[1], fb[1]);
    mfma_step(fa[0], fl[0], fb[0]);
#pragma unroll
    for (int i = 0; i < NDS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
    __builtin_amdgcn_sched_barrier(0);
    // step 1: stage kt+1 must have landed (own loads, then the barrier for everyone else's).
    // Past the barrier every wave holds stage kt's last fragments in registers, so its slot is
    // refilled right away with stage kt+S: each load has S-1 whole iterations to land.  The
    // fragment reads are issued before the loads into LDS: the compiler cannot prove that the
    // two touch different stages, so reads placed after the loads could not move past them
    // and the loads would issue as one burst instead of one per MFMA.
    wait_vm<(S - 2) * G::LPW>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    lfrag((kt + 1) % S, 0, fa[0], fl[0], fb[0]);
    issue(kt + S, buf);
    mfma_step(fa[1], fl[1], fb[1]);
    // Three fragment reads per MFMA, then one load per MFMA: the loads into LDS must follow
    // every fragment read (see above), and spreading them one per MFMA keeps the vector memory
    // queue from filling behind a burst, which would hold up the wave's next MFMAs.  Tiles with
    // too few MFMAs for that take the reads and the loads each in one group.
    {
      constexpr int ND3 = (NDS + 2) / 3;
      if constexpr (ND3 + G::LPW <= NMF) {
#pragma unroll
        for (int i = 0; i < ND3; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // DS read
        }
#pragma unroll
        for (int i = 0; i < G::LPW; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read (buffer load -> LDS)
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, G::LPW, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  }
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
  // drain the (redundant) trailing loads before the ring is reused for the epilogue
  wait_vm<0>();
  __syncthreads();

  // ---- epilogue through LDS, one 32-row slice of the wave tile at a time, in a region only
  // this wave touches (LDS operations of one wave complete in order, so no barrier is needed
  // between slices).  Accumulator layout: lane holds column (lane & 31) and rows
  // 8g + 4*(lane >> 5) + e of each 32x32 tile.
  float* sc = reinterpret_cast<float*>(smem) + wv * 32 * G::SST;
  const int lc = lane & 31, lr = (lane >> 5) * 4;
  // AM 3: the float16 weights carry a power-of-two scale; undoing it is exact
  const float osc = AM == 3 ? p.acc_scale : 1.0f;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sc[(8 * (e / 4) + lr + (e % 4)) * G::SST + j * 32 + lc] = AM == 3 ? acc[i][j][e] * osc : acc[i][j][e];
    epilogue_slice<EPI, TN * 32, AM>(p, M, sc, m0 + wm * TM * 32 + i * 32, n0 + wn * TN * 32, lane);
  }
}

// Tile configurations (2x2 or 2x1 waves):
//   L 256x256 (waves of 128x128), T 192x256 (96x128), H 128x256 (64x128), S 64x64 (2 waves of
//   32x64), one workgroup per CU; O 128x256 with two workgroups per CU, so one workgroup's
//   epilogue (residual read-modify-write, activation stores) runs under the other's main loop.
enum Cfg { CFG_L, CFG_T, CFG_H, CFG_O, CFG_S };
struct CfgInfo {
  int cfg, bm, bn, wave_n, occ;
  double eff;   // relative efficiency (larger wave tiles read less LDS per MFMA)
};
// (efficiencies fitted to measured times of the tower's products on MI355X)
constexpr CfgInfo kCfgs[] = {{CFG_L, 256, 256, 128, 1, 1.0},   // (order used by pick_cfg)
                             {CFG_T, 192, 256, 128, 1, 0.98},
                             {CFG_H, 128, 256, 128, 1, 0.9},
                             {CFG_O, 128, 256, 128, 2, 1.1},
                             {CFG_S, 64, 64, 64, 1, 0.3}};

template <int BM, int BN, int WM, int WN, int AM, int EPI, int OCC = 1>
hipError_t run(const GemmArgs& a, hipStream_t st) {
  using G = Geo<BM, BN, WM, WN, AM, OCC>;
  const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (a.m_dev)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, AM, EPI, OCC, true>), dim3((unsigned)tiles), dim3(G::NT),
                       G::kSmem, st, a);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, AM, EPI, OCC, false>), dim3((unsigned)tiles), dim3(G::NT),
                       G::kSmem, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int AM, int EPI, int OCC = 1>
hipError_t allow_smem() {
  using G = Geo<BM, BN, WM, WN, AM, OCC>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel<BM, BN, WM, WN, AM, EPI, OCC, false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, G::kSmem);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel<BM, BN, WM, WN, AM, EPI, OCC, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, G::kSmem);
  return e;
}

template <int AM, int EPI>
hipError_t allow_smem_all() {
  hipError_t e = allow_smem<256, 256, 2, 2, AM, EPI>();
  if (e == hipSuccess) e = allow_smem<192, 256, 2, 2, AM, EPI>();
  if (e == hipSuccess) e = allow_smem<128, 256, 2, 2, AM, EPI>();
  if (e == hipSuccess) e = allow_smem<128, 256, 2, 2, AM, EPI, 2>();
  if (e == hipSuccess) e = allow_smem<64, 64, 2, 1, AM, EPI>();
  return e;
}

template <int AM, int EPI>
hipError_t run_cfg(int cfg, const GemmArgs& a, hipStream_t st) {
  switch (cfg) {
    case CFG_L: return run<256, 256, 2, 2, AM, EPI>(a, st);
    case CFG_T: return run<192, 256, 2, 2, AM, EPI>(a, st);
    case CFG_H: return run<128, 256, 2, 2, AM, EPI>(a, st);
    case CFG_O: return run<128, 256, 2, 2, AM, EPI, 2>(a, st);
    default: return run<64, 64, 2, 1, AM, EPI>(a, st);
  }
}

// Estimated time ~ rounds of (256 * occupancy) workgroups x per-CU area of a round / efficiency.
static_assert(kCfgs[1].cfg == CFG_T && kCfgs[3].cfg == CFG_O, "pick_cfg indexes the table");

int pick_cfg(int epi, const GemmArgs& a) {
  auto fits = [&](const CfgInfo& c) {
    return a.N % c.bn == 0 && !(epi == EPI_QKV && a.hidden % c.wave_n);   // QKV: a wave's columns stay in one of q / k / v
  };
  auto tiles_of = [&](const CfgInfo& c) { return (double)((a.M + c.bm - 1) / c.bm) * (a.N / c.bn); };
  // Measured on the tower's products with blocked operands: two workgroups per CU win as
  // soon as every CU gets a tile (each hides the other's epilogue and barriers), except for
  // long reductions where the 192x256 tile already fills >= 85% of its last round.
  const CfgInfo& o = kCfgs[3];
  const CfgInfo& t = kCfgs[1];
  if (fits(o) && tiles_of(o) >= 256.0) {
    const int k_eff = a.K * (a.a_group > 0 || a.A8 ? 2 : 1);   // compensated products: two MFMA passes' worth
    const double t_fill = tiles_of(t) / (256.0 * std::ceil(tiles_of(t) / 256.0));
    if (k_eff >= 8192 && fits(t) && t_fill >= 0.85) return t.cfg;
    return o.cfg;
  }
  int best = -1;
  double best_t = 1e300;
  for (const CfgInfo& c : kCfgs) {
    if (!fits(c)) continue;
    const double tiles = tiles_of(c);
    const double rounds = std::ceil(tiles / (256.0 * c.occ));
    // co-resident workgroups only hide each other's epilogues once they are staggered,
    // i.e. from the second round on; a single round runs like one workgroup per CU
    const double eff = (c.occ > 1 && rounds < 2) ? 0.9 : c.eff;
    const double t = rounds * c.occ * c.bm * c.bn / eff;
    if (t < best_t) {
      best_t = t;
      best = c.cfg;
    }
  }
  return best;
}

template <int AM>
hipError_t dispatch(int epi, int cfg, const GemmArgs& a, hipStream_t st, bool* bad_epi) {
  switch (epi) {
    case EPI_F32:   // (patch embedding only, always bf16: not built for the other modes)
      if constexpr (AM == 2 || AM == 3) break;
      else return run_cfg<AM, EPI_F32>(cfg, a, st);
    case EPI_RES: return run_cfg<AM, EPI_RES>(cfg, a, st);
    case EPI_GELU: return run_cfg<AM, EPI_GELU>(cfg, a, st);
    case EPI_SWIGLU: return run_cfg<AM, EPI_SWIGLU>(cfg, a, st);
    case EPI_QKV: return run_cfg<AM, EPI_QKV>(cfg, a, st);
    case EPI_OUT: return run_cfg<AM, EPI_OUT>(cfg, a, st);
    default: break;
  }
  *bad_epi = true;
  return hipSuccess;
}

template <int AM>
hipError_t allow_all() {
  hipError_t e = hipSuccess;
  if constexpr (AM != 2 && AM != 3) e = allow_smem_all<AM, EPI_F32>();
  if (e == hipSuccess) e = allow_smem_all<AM, EPI_RES>();
  if (e == hipSuccess) e = allow_smem_all<AM, EPI_GELU>();
  if (e == hipSuccess) e = allow_smem_all<AM, EPI_SWIGLU>();
  if (e == hipSuccess) e = allow_smem_all<AM, EPI_QKV>();
  if (e == hipSuccess) e = allow_smem_all<AM, EPI_OUT>();
  return e;
}

}  // namespace

vit_status prepare_gemm_kernels() {
  hipError_t e = allow_all<0>();
  if (e == hipSuccess) e = allow_all<1>();
  if (e == hipSuccess) e = allow_all<2>();
  if (e == hipSuccess) e = allow_all<3>();
  if (e != hipSuccess) {
    set_error("gemm LDS attribute: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

vit_status launch_gemm(int epi, const GemmArgs& in, void* stream) {
  if (in.M <= 0) return VIT_OK;
  GemmArgs a = in;
  const bool split = a.a_group > 0;
  const bool f8 = a.A8 != nullptr;
  const int64_t a_cols = split ? 2 * (int64_t)a.K : a.K;
  const bool bf16_out = epi == EPI_GELU || epi == EPI_SWIGLU;
  if (a.N % 64 || a.K % BK || a.K <= 0 || a.lda % BK || a.ldb % BK || a.lda < a_cols || a.ldb < a.K ||
      a.ldo % 4 || (bf16_out && (a.ldo % BK || a.split_off % BK)) ||
      (split && (a.a_group % BK || a.K % a.a_group))) {
    set_error("gemm: unsupported shape M=%d N=%d K=%d group=%d (N a multiple of 64; K, the hi/lo group and "
              "the blocked operand widths multiples of 32)", a.M, a.N, a.K, a.a_group);
    return VIT_E_ARG;
  }
  if (f8 && (split || !a.B8 || !a.b8_scale || a.K % 64 || a.lda8 % BK || a.ldb8 % BK || a.lda8 < a.K ||
             a.ldb8 < a.K || (bf16_out && (!a.out8 || a.ldo8 % BK)) || (!bf16_out && a.out8) || epi == EPI_F32)) {
    set_error("gemm: e4m3 residual operands need B8, its scales, K a multiple of 64, fp8 widths multiples of 32 "
              "and an e4m3 output exactly for the GELU / SwiGLU epilogues (M=%d N=%d K=%d epi %d)", a.M, a.N,
              a.K, epi);
    return VIT_E_ARG;
  }
  if (!f8 && a.out8) {
    set_error("gemm: an e4m3 residual output needs e4m3 residual inputs");
    return VIT_E_ARG;
  }
  if (a.f16 && (f8 || split || a.split_off)) {
    set_error("gemm: float16 operands take no compensation");
    return VIT_E_ARG;
  }
  // byte extents of the blocked operands (rows padded to 16), addressed with 32-bit buffer offsets
  const int64_t a_bytes = round_up(a.M, 16) * a.lda * 2;
  const int64_t b_bytes = (int64_t)a.N * a.ldb * 2;
  if (a_bytes >= (int64_t)1 << 31 || b_bytes >= (int64_t)1 << 31) {
    set_error("gemm: operand larger than 2 GiB (M=%d N=%d K=%d)", a.M, a.N, a.K);
    return VIT_E_ARG;
  }
  a.a_bytes = (uint32_t)a_bytes;
  a.b_bytes = (uint32_t)b_bytes;
  if (f8) {   // e4m3 rows padded to 32
    const int64_t a8 = round_up(a.M, 32) * a.lda8, b8 = (int64_t)a.N * a.ldb8;
    if (a8 >= (int64_t)1 << 31 || b8 >= (int64_t)1 << 31) {
      set_error("gemm: e4m3 operand larger than 2 GiB (M=%d N=%d K=%d)", a.M, a.N, a.K);
      return VIT_E_ARG;
    }
    a.a8_bytes = (uint32_t)a8;
    a.b8_bytes = (uint32_t)b8;
  }
  const int cfg = pick_cfg(epi, a);
  if (cfg < 0) {
    set_error("gemm: no tile configuration for N=%d (epilogue %d)", a.N, epi);
    return VIT_E_ARG;
  }
  // Tile grouping: 8 row tiles deep, except for one-workgroup-per-CU tiles over few column
  // tiles, where a group holds as many whole row panels as an XCD runs at once (32
  // workgroups), so every column tile of a panel reads it from L2 at about the same time
  // (fc2-shaped product: 407 -> 393 us).
  const CfgInfo* ci = nullptr;
  for (const CfgInfo& c : kCfgs)
    if (c.cfg == cfg) ci = &c;
  const int gn = a.N / ci->bn;
  a.group_m = (ci->occ == 1 && gn <= 8) ? std::max(1, 32 / gn) : 8;
  hipStream_t st = static_cast<hipStream_t>(stream);
  bool bad_epi = false;
  const hipError_t e = f8       ? dispatch<2>(epi, cfg, a, st, &bad_epi)
                      : split  ? dispatch<1>(epi, cfg, a, st, &bad_epi)
                      : a.f16  ? dispatch<3>(epi, cfg, a, st, &bad_epi)
                               : dispatch<0>(epi, cfg, a, st, &bad_epi);
  if (bad_epi) {
    set_error("gemm: bad epilogue %d", epi);
    return VIT_E_ARG;
  }
  if (e != hipSuccess) {
    set_error("gemm launch (epi %d, M=%d N=%d K=%d): %s", epi, a.M, a.N, a.K, hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

}  // namespace vitmi
