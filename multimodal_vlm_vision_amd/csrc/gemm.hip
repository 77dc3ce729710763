// bf16 MFMA GEMM for gfx950 with fused epilogues.
//
// C[M][N] = A[M][K] * B[N][K]^T: both operands are K-contiguous (activations
// row-major, weights stored [out, in]), fp32 accumulation in
// v_mfma_f32_32x32x16_bf16.  Used for every dense product of the tower:
// patch embedding (the stride = kernel 3D conv as one GEMM, "vLLM multimodal
// inference | ViT performance optimisation", section 3.2), qkv, out-proj,
// MLP and the merger MLP (sections 2.2 and 3.1).  The small elementwise steps
// that follow a product are fused into its epilogue (section 3.5): bias,
// exact-erf GELU, SiLU(gate)*up, residual add into the fp32 stream, the 2D
// RoPE of q and k (section 3.3), and the merger's row scatter.
//
// Main loop: BM x BN workgroup tile, BK = 64, WM x WN waves, each wave owning
// (BM/WM) x (BN/WN) as 32x32 MFMA tiles.  Tiles move global -> LDS with
// gfx950's direct loads (global_load_lds_dwordx4: no VGPR staging, no
// ds_write), double-buffered; each wave's 1 KB load covers 8 tile rows and
// its lanes fetch the 16-byte chunks in the XOR-swizzled order the fragment
// reads expect (chunk ^ ((row >> 1) & 7), so 16 consecutive rows hit
// distinct banks).  MFMA operand fragments are double-buffered in registers
// one 16-wide K step ahead.  Workgroups are remapped so each XCD (dispatch is
// round-robin over 8 XCDs) runs a contiguous range of tiles, grouped 8
// row-tiles deep, to keep A and B panels in its L2.
//
// Epilogue: the accumulators are staged through LDS one 32-row slice at a
// time, so every global access of the epilogue is a 16-byte (fp32) or 8-byte
// (bf16) vector: residual read-modify-write, bias, activations, RoPE pairs
// and the transposed V store all run on 4 consecutive columns (or rows).
#include <hip/hip_runtime.h>

#include <cmath>

#include "vit_internal.h"

namespace vitmi {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BK = 64;
constexpr int kGroupM = 8;

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

__device__ __forceinline__ uint2 pack4(float4 v) { return make_uint2(pack2(v.x, v.y), pack2(v.z, v.w)); }

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

// bf16 activation store: hi = bf16(y) at column n; with split_off, lo = bf16(y - hi) at n + split_off
__device__ __forceinline__ void store_act(const GemmArgs& p, int m, int n, float4 y) {
  uint16_t* o = static_cast<uint16_t*>(p.out) + (int64_t)m * p.ldo + n;
  const uint2 hi = pack4(y);
  *reinterpret_cast<uint2*>(o) = hi;
  if (p.split_off) {
    const float4 h = make_float4(__builtin_bit_cast(float, hi.x << 16), __builtin_bit_cast(float, hi.x & 0xffff0000u),
                                 __builtin_bit_cast(float, hi.y << 16), __builtin_bit_cast(float, hi.y & 0xffff0000u));
    *reinterpret_cast<uint2*>(o + p.split_off) = pack4(make_float4(y.x - h.x, y.y - h.y, y.z - h.z, y.w - h.w));
  }
}

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int kStage = (BM + BN) * BK;            // elements per LDS stage
  static constexpr int LPW = (BM + BN) / 8 / NW;            // 1 KB direct loads per wave per stage
  static constexpr int SST = TN * 32 + 8;                   // epilogue slice row stride (floats)
  static constexpr size_t kStageBytes = 2 * (size_t)kStage * 2;       // double-buffered stages
  static constexpr size_t kSliceBytes = (size_t)NW * 32 * SST * 4;    // one fp32 slice per wave
  static constexpr size_t kSmem = kStageBytes > kSliceBytes ? kStageBytes : kSliceBytes;
  static_assert(TM >= 1 && TN >= 2 && TN % 2 == 0, "wave tile must hold column pairs");
  static_assert((BM + BN) % (8 * NW) == 0, "direct-load split");
  static_assert(kSmem <= 160 * 1024, "LDS budget");
};

// Applies the epilogue to one staged 32-row slice (rows m_base.., columns n_base.., width W = TN*32).
template <int EPI, int W>
__device__ __forceinline__ void epilogue_slice(const GemmArgs& p, const float* sc, int m_base, int n_base,
                                               int lane) {
  constexpr int SST = W + 8;
  constexpr int C4 = W / 4;   // float4 chunks per row
  if (EPI == EPI_F32 || EPI == EPI_RES || EPI == EPI_GELU || EPI == EPI_OUT) {
#pragma unroll
    for (int q = 0; q < 32 * C4 / 64; ++q) {
      const int id = lane + 64 * q, r = id / C4, c4 = id % C4;
      const int m = m_base + r, n = n_base + 4 * c4;
      if (m >= p.M) continue;
      const float4 v = *reinterpret_cast<const float4*>(sc + r * SST + 4 * c4);
      if (EPI == EPI_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (int64_t)m * p.ldo + n) = v;
      } else {
        const float4 b = *reinterpret_cast<const float4*>(p.bias + n);
        if (EPI == EPI_RES) {
          float4* o = reinterpret_cast<float4*>(static_cast<float*>(p.out) + (int64_t)m * p.ldo + n);
          *o = f4add(*o, f4add(v, b));
        } else if (EPI == EPI_OUT) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (int64_t)p.row_map[m] * p.ldo + n) = f4add(v, b);
        } else {   // GELU -> bf16 (hi, and lo when split)
          const float4 x = f4add(v, b);
          store_act(p, m, n, make_float4(gelu(x.x), gelu(x.y), gelu(x.z), gelu(x.w)));
        }
      }
    }
  } else if (EPI == EPI_SWIGLU || (EPI == EPI_QKV && n_base < 2 * p.hidden)) {
    // pairs: columns c (c % 64 < 32) and c + 32 of each 64-column block
    constexpr int G4 = W / 8;   // first-member float4 chunks per row
#pragma unroll
    for (int q = 0; q < 32 * G4 / 64; ++q) {
      const int id = lane + 64 * q, r = id / G4, g = id % G4;
      const int cl = (g / 8) * 64 + (g % 8) * 4;          // local column of the first member
      const int m = m_base + r, n = n_base + cl;
      if (m >= p.M) continue;
      const float4 a = f4add(*reinterpret_cast<const float4*>(sc + r * SST + cl),
                             *reinterpret_cast<const float4*>(p.bias + n));
      const float4 b = f4add(*reinterpret_cast<const float4*>(sc + r * SST + cl + 32),
                             *reinterpret_cast<const float4*>(p.bias + n + 32));
      if (EPI == EPI_SWIGLU) {
        const int oc = (n - (n & 63)) / 2 + (n & 31);
        const float4 y = make_float4(silu(a.x) * b.x, silu(a.y) * b.y, silu(a.z) * b.z, silu(a.w) * b.w);
        store_act(p, m, oc, y);
      } else {
        // RoPE on 4 consecutive rotary pairs of one head (head_dim/2 is a multiple of 4)
        const int d = p.hidden, hd = p.head_dim, rr = hd / 2, nf = p.nfreq;
        const int part = n / d, jj = n - part * d;
        const int pair = 32 * (jj / 64) + (jj % 64);
        const int head = pair / rr, kk = pair % rr;
        const int pos = p.row_pos[m];
        const int ax = kk < nf ? (pos >> 16) : (pos & 0xffff);
        const int fi = kk < nf ? kk : kk - nf;
        const float4 cs = *reinterpret_cast<const float4*>(p.cos_tab + ax * nf + fi);
        const float4 sn = *reinterpret_cast<const float4*>(p.sin_tab + ax * nf + fi);
        const float4 y1 = make_float4(a.x * cs.x - b.x * sn.x, a.y * cs.y - b.y * sn.y,
                                      a.z * cs.z - b.z * sn.z, a.w * cs.w - b.w * sn.w);
        const float4 y2 = make_float4(b.x * cs.x + a.x * sn.x, b.y * cs.y + a.y * sn.y,
                                      b.z * cs.z + a.z * sn.z, b.w * cs.w + a.w * sn.w);
        uint16_t* o = (part == 0 ? p.q : p.k) + ((int64_t)head * p.n_tok + m) * hd;
        *reinterpret_cast<uint2*>(o + kk) = pack4(y1);
        *reinterpret_cast<uint2*>(o + kk + rr) = pack4(y2);
      }
    }
  } else if (EPI == EPI_QKV) {
    // V part: transposed store [head][dim][token]; each item is 4 consecutive rows of one column
    const int d = p.hidden, hd = p.head_dim;
#pragma unroll
    for (int q = 0; q < 8 * W / 64; ++q) {
      const int id = lane + 64 * q, rg = id % 8, c = id / 8;
      const int m = m_base + 4 * rg, n = n_base + c;
      if (m >= p.M) continue;
      const float b = p.bias[n];
      const float4 v = make_float4(sc[(4 * rg + 0) * SST + c] + b, sc[(4 * rg + 1) * SST + c] + b,
                                   sc[(4 * rg + 2) * SST + c] + b, sc[(4 * rg + 3) * SST + c] + b);
      const int nn = n - 2 * d, head = nn / hd, dd = nn % hd;
      *reinterpret_cast<uint2*>(p.vt + ((int64_t)head * hd + dd) * p.n_tok + m) = pack4(v);
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(GemmArgs p) {
  using T = Tile<BM, BN, WM, WN>;
  constexpr int TM = T::TM, TN = T::TN, LPW = T::LPW, SST = T::SST;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv % WM, wn = wv / WM;

  // ---- tile index: XCD-contiguous ranges, then grouped row-major order
  const int gm = (p.M + BM - 1) / BM, gn = (p.N + BN - 1) / BN;
  const int G = gm * gn;
  const int pid = blockIdx.x;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + local;
  const int in_group = kGroupM * gn;
  const int grp = logical / in_group, first_m = grp * kGroupM;
  const int gsz = min(gm - first_m, kGroupM);
  const int li = logical % in_group;
  const int m0 = (first_m + li % gsz) * BM, n0 = (li / gsz) * BN;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // direct-load sources: wave wv fills stage rows [(wv*LPW + j)*8, +8); lane -> row lane/8,
  // physical chunk lane%8, which holds logical chunk (lane%8) ^ ((row >> 1) & 7).
  // Rows past M / N read the last valid row; those results are never stored.
  const uint16_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = (wv * LPW + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    src[j] = r < BM ? p.A + (int64_t)min(m0 + r, p.M - 1) * p.lda + c * 8
                    : p.B + (int64_t)min(n0 + r - BM, p.N - 1) * p.ldb + c * 8;
  }
  auto dload = [&](int kt, int buf) {
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src[j] + kt * BK),
          (__attribute__((address_space(3))) void*)(smem + buf * T::kStage + (wv * LPW + j) * 8 * BK), 16, 0, 0);
  };
  bf16x8 fa[2][TM], fb[2][TN];
  auto lfrag = [&](int buf, int kk, bf16x8 (&xa)[TM], bf16x8 (&xb)[TN]) {
    const uint16_t* sA = smem + buf * T::kStage;
    const uint16_t* sB = sA + BM * BK;
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * TM * 32 + i * 32 + (lane & 31);
      xa[i] = *reinterpret_cast<const bf16x8*>(sA + r * BK + swz(r, c) * 8);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * TN * 32 + j * 32 + (lane & 31);
      xb[j] = *reinterpret_cast<const bf16x8*>(sB + r * BK + swz(r, c) * 8);
    }
  };

  const int nk = p.K / BK;
  dload(0, 0);
  __syncthreads();
  lfrag(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) dload(kt + 1, cur ^ 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int s = kk & 1;
      if (kk < BK / 16 - 1) lfrag(cur, kk + 1, fa[s ^ 1], fb[s ^ 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) lfrag(cur ^ 1, 0, fa[0], fb[0]);
  }

  // ---- epilogue through LDS, one 32-row slice of the wave tile at a time.  Accumulator
  // layout: lane holds column (lane & 31) and rows 8g + 4*(lane >> 5) + e of each 32x32 tile.
  float* sc = reinterpret_cast<float*>(smem) + wv * 32 * SST;
  const int lc = lane & 31, lr = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i > 0) __syncthreads();
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[(8 * (e / 4) + lr + (e % 4)) * SST + j * 32 + lc] = acc[i][j][e];
    __syncthreads();
    epilogue_slice<EPI, TN * 32>(p, sc, m0 + wm * TM * 32 + i * 32, n0 + wn * TN * 32, lane);
  }
}

// Tile configurations: L 256x256 (8 waves of 64x128), M 128x128 (4 waves of 64x64),
// S 64x64 (2 waves of 32x64).
enum Cfg { CFG_L, CFG_M, CFG_S };
struct CfgInfo {
  int cfg, bm, bn, wave_n;
  double eff;   // measured relative MFMA efficiency of the main loop
};
constexpr CfgInfo kCfgs[] = {{CFG_L, 256, 256, 128, 1.0}, {CFG_M, 128, 128, 64, 0.85}, {CFG_S, 64, 64, 64, 0.35}};

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t run(const GemmArgs& a, hipStream_t st) {
  using T = Tile<BM, BN, WM, WN>;
  const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI>), dim3((unsigned)tiles), dim3(T::NT), T::kSmem, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t allow_smem() {
  using T = Tile<BM, BN, WM, WN>;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel<BM, BN, WM, WN, EPI>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)T::kSmem);
}

template <int EPI>
hipError_t allow_smem_all() {
  hipError_t e = allow_smem<256, 256, 4, 2, EPI>();
  if (e == hipSuccess) e = allow_smem<128, 128, 2, 2, EPI>();
  if (e == hipSuccess) e = allow_smem<64, 64, 2, 1, EPI>();
  return e;
}

template <int EPI>
hipError_t run_cfg(int cfg, const GemmArgs& a, hipStream_t st) {
  switch (cfg) {
    case CFG_L: return run<256, 256, 4, 2, EPI>(a, st);
    case CFG_M: return run<128, 128, 2, 2, EPI>(a, st);
    default: return run<64, 64, 2, 1, EPI>(a, st);
  }
}

// Estimated time ~ rounds of 256 workgroups x tile area / relative efficiency.
int pick_cfg(int epi, const GemmArgs& a) {
  int best = -1;
  double best_t = 1e300;
  for (const CfgInfo& c : kCfgs) {
    if (a.N % c.bn) continue;
    if (epi == EPI_QKV && (a.hidden % c.wave_n)) continue;   // a wave's columns stay in one of q / k / v
    const double tiles = (double)((a.M + c.bm - 1) / c.bm) * (a.N / c.bn);
    const double t = std::ceil(tiles / 256.0) * c.bm * c.bn / c.eff;
    if (t < best_t) {
      best_t = t;
      best = c.cfg;
    }
  }
  return best;
}

}  // namespace

vit_status prepare_gemm_kernels() {
  hipError_t e = allow_smem_all<EPI_F32>();
  if (e == hipSuccess) e = allow_smem_all<EPI_RES>();
  if (e == hipSuccess) e = allow_smem_all<EPI_GELU>();
  if (e == hipSuccess) e = allow_smem_all<EPI_SWIGLU>();
  if (e == hipSuccess) e = allow_smem_all<EPI_QKV>();
  if (e == hipSuccess) e = allow_smem_all<EPI_OUT>();
  if (e != hipSuccess) {
    set_error("gemm LDS attribute: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

vit_status launch_gemm(int epi, const GemmArgs& a, void* stream) {
  if (a.M <= 0) return VIT_OK;
  if (a.N % 64 || a.K % BK || a.K <= 0 || a.lda % 8 || a.ldb % 8 || a.ldo % 4) {
    set_error("gemm: unsupported shape M=%d N=%d K=%d (N, K must be multiples of 64)", a.M, a.N, a.K);
    return VIT_E_ARG;
  }
  const int cfg = pick_cfg(epi, a);
  if (cfg < 0) {
    set_error("gemm: no tile configuration for N=%d (epilogue %d)", a.N, epi);
    return VIT_E_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (epi) {
    case EPI_F32: e = run_cfg<EPI_F32>(cfg, a, st); break;
    case EPI_RES: e = run_cfg<EPI_RES>(cfg, a, st); break;
    case EPI_GELU: e = run_cfg<EPI_GELU>(cfg, a, st); break;
    case EPI_SWIGLU: e = run_cfg<EPI_SWIGLU>(cfg, a, st); break;
    case EPI_QKV: e = run_cfg<EPI_QKV>(cfg, a, st); break;
    case EPI_OUT: e = run_cfg<EPI_OUT>(cfg, a, st); break;
    default:
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
