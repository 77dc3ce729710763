// Block-diagonal (varlen) flash attention for the vision tower on gfx950.
//
// For every segment s and head h: O_s = softmax(Q_s K_s^T / sqrt(head_dim)) V_s,
// with segments = items (cu_seqlens; attention never crosses an image
// boundary: "vLLM multimodal inference | ViT performance optimisation",
// section 3.4) or, in window-attention layers, windows laid out contiguously
// by the planner (section 3.3).  A tile never spans two segments: every work
// unit names its segment and the kernel only reads that segment's keys.
//
// Formulation (v_mfma_f32_32x32x16_f16 throughout with float16 operands, the
// default; _bf16 with bfloat16 ones): a wave owns 64 queries as two 32-query
// tiles and walks the segment's keys 32 at a time.
//  * S^T = K Q^T: keys are MFMA rows, queries columns, head_dim the reduction
//    (80 = 5 x 16, no padded chunk).  Each lane ends up with 16 keys
//    (rows 8g + 4h + e, h = lane / 32) of one query (lane % 32), so the row
//    max is 15 in-lane maxima and one permlane32 swap with the lane holding
//    the other 16 keys.
//  * O^T = V^T P^T: the lane's 16 probabilities are directly its B operands
//    for the two 16-key reduction chunks (chunk c takes rows g = 2c, 2c + 1);
//    with K rows loaded in key_at order those are keys 16c + 8h + 0..7, so
//    each V^T fragment is one 16-byte chunk of a V^T row.  P never leaves
//    registers.
//  * The softmax denominator comes from the padding of the last O^T row tile:
//    row head_dim of the V^T tile holds ones (and the rows after it zeros), so
//    O^T row head_dim accumulates sum_k P.
// Online softmax in fp32 with exp2: q arrives scaled by log2(e)/sqrt(d) (the
// qkv epilogue applies it before q is rounded to 16 bits), and every score MFMA
// chain starts from an accumulator tile holding -m (the query's running
// offset), so the MFMAs return the exp2 argument s - m itself and the common
// path spends no VALU op on it; P is rounded to the operand type for the MFMA.  The offset
// is only raised (and O rescaled) when a block's max exceeds it by more than
// 2^8, which keeps the rescale off the common path without changing the math.
// A block's score MFMAs, and its softmax up to the last tile's exponentials, run
// at raised wave priority (s_setprio): a co-resident wave then fills the matrix
// pipe's gaps instead of delaying the chain from the scores to the probabilities
// (raising the P.V MFMAs as well measured slower on long segments).  The score
// MFMAs' K fragments are read three ahead of their MFMAs.
//
// K tiles (32 keys x head_dim, row stride head_dim + 8 so 16-byte fragment
// reads of 16 consecutive rows hit distinct banks; keys in the row order of
// key_at, which makes each lane's probabilities 8 consecutive keys) and V^T
// tiles (head_dim rows x the block's 32 keys, 16-byte chunks rotated by row
// bits 2-3, so a P.V fragment is one conflict-free 16-byte read) move
// global -> LDS with gfx950's 16-byte buffer loads into LDS, into a ring of
// two stages (of two key blocks per stage and one workgroup barrier per stage
// for the 4-wave workgroups, one block per stage for the 1-wave ones).  Work
// units are laid out so each XCD
// (workgroups are dispatched round-robin over 8 XCDs) runs contiguous
// (head, segment) ranges and shares their K/V in its L2.  Long segments use
// 4-wave workgroups (256 queries share each K/V tile); short segments
// (windows) use 1-wave workgroups of 64 queries.  The DYN instantiations read
// the work-list length from device memory (bucketed graphs: the grid covers the
// capacity and surplus workgroups leave at once).  The PART instantiation runs
// the planner's key-split lists: a unit may cover only a range of its query
// block's key blocks, leaving its unnormalised output, running offset and
// denominator in a partial slot that attn_merge_kernel combines.
#include <hip/hip_runtime.h>

#include <cmath>

#include "vit_internal.h"

namespace vitmi {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int KB = 32;   // keys per step
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit dword format, no swizzle
constexpr int QT = 2;    // 32-query tiles per wave (64 queries)

// the value held by lanes l and l ^ 32: both halves of x are swapped into place in registers
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}
// x of lane l & 31 (lower half) in every lane
__device__ __forceinline__ float from_lower_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, r[0]);
}
// x of lane (l & 31) + 32 (upper half) in every lane
__device__ __forceinline__ float from_upper_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, r[1]);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// two floats -> packed float16 pair, round to nearest even (one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// F16: q, k, V^T, P and the output are float16 (the default activation form); otherwise bfloat16.
// Operand fragments travel as 16-byte vectors of either type (same bits, same layout).
template <bool F16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (F16) return pack_f16(a, b);
  else return pack_bf16(a, b);
}
template <bool F16>
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// x - bf16(x): what the bf16 rounding of x leaves out
__device__ __forceinline__ float bf16_rest(float x) { return x - (float)(__bf16)x; }

// four residuals x - bf16(x), times 2^kLoShift and clamped to e4m3's finite range, as four OCP
// e4m3 bytes (round to nearest even): the compensated-activation format the GEMMs read
__device__ __forceinline__ uint32_t rest_e4m3x4(float a, float b, float c, float d) {
  constexpr float s = (float)(1 << kLoShift);
  auto f = [](float x) { return fminf(fmaxf(bf16_rest(x) * s, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f(a), f(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f(c), f(d), lo, true);
}

// Key of row p of a block's K tile.  S^T = K Q^T leaves lane (query, h) with rows
// 8g + 4h + e (g, e < 4) of the 32-row score tile; loading key 16c + 8h + 4b + e into row
// 16c + 8b + 4h + e makes the lane's probabilities of reduction chunk c (g = 2c, 2c + 1) the
// eight consecutive keys 16c + 8h + 0..7 -- in the order the P.V MFMA pairs them with one
// 16-byte V^T chunk.  Rows past 32 (the padding loads) keep their index.
__device__ __forceinline__ int key_at(int p) {
  return p < 32 ? (p & 0x13) | ((p & 4) << 1) | ((p & 8) >> 1) : p;
}

// Four consecutive output columns of one row, in the blocked GEMM layout (the out-projection's
// A operand): the rounded values, plus what their bf16 rounding leaves out when the
// out-projection compensates it (hi+lo rows or an e4m3 residual).  (The attention kernel's own
// epilogue writes the same forms inline.)
template <bool F16>
__device__ __forceinline__ void store_o4(const AttnArgs& a, int64_t orow, int col, float y0, float y1, float y2,
                                         float y3) {
  const int hid = a.heads * a.head_dim;
  const int ld = a.o_split ? 2 * hid : hid;
  *reinterpret_cast<uint2*>(a.o + kt_index(orow, col, ld)) = make_uint2(pack16<F16>(y0, y1), pack16<F16>(y2, y3));
  if (F16) return;   // float16 output needs no compensation
  if (a.o_split)
    *reinterpret_cast<uint2*>(a.o + kt_index(orow, hid + col, ld)) =
        make_uint2(pack_bf16(bf16_rest(y0), bf16_rest(y1)), pack_bf16(bf16_rest(y2), bf16_rest(y3)));
  if (a.o8) *reinterpret_cast<uint32_t*>(a.o8 + kt8_index(orow, col, hid)) = rest_e4m3x4(y0, y1, y2, y3);
}

// DYN: the work-list length comes from device memory at run time (bucketed graphs); a separate
// instantiation, so the plain path keeps it a launch constant.
template <int HD, int NW, bool DYN, bool F16, bool PART>
__global__ void __launch_bounds__(NW * 64, 2)
attn_kernel(AttnArgs a, const AttnWork* __restrict__ work, int n_work, const int32_t* __restrict__ n_work_dev) {
  constexpr int NCH = HD / 16;               // 16-wide reduction chunks of S^T = K Q^T
  constexpr int DT = (HD + 1 + 31) / 32;     // 32-row tiles of O^T, incl. the row of ones
  constexpr int KS = HD + 8;                 // K tile row stride (elements)
  constexpr int KCH = KS / 8;                // 16-byte chunks per K row (the last is padding)
  constexpr int KLOADS = (KB * KCH + 63) / 64;      // 1 KB direct loads per K tile
  // V^T tile: each row holds the block's 32 keys (4 chunks of 8 keys), its chunks rotated by
  // bits 2-3 of the row (chunk q at q ^ ((row >> 2) & 3)), so that a fragment read -- one 16-byte
  // chunk of 32 consecutive rows -- touches every bank once per 16 lanes.
  constexpr int VP = KB;                     // keys per V^T tile row (64 bytes, 4 chunks)
  constexpr int VCH = VP / 8;                // 16-byte chunks per V^T row
  constexpr int VDW = VP / 2;                // dwords per V^T row
  constexpr int VROWS = DT * 32;             // rows HD.. are constant (ones, then zeros)
  constexpr int VLOADS = (HD * VCH + 63) / 64;      // 1 KB direct loads per V^T tile
  constexpr int LROW = HD - 32 * (DT - 1);   // row of the sums inside the last O^T tile
  constexpr int LIDX = 4 * (LROW / 8) + (LROW % 4), LHALF = (LROW % 8) / 4;
  static_assert(HD % 16 == 0 && KCH % 2 == 1, "head_dim must be a multiple of 16");

  // Ring slots as separate objects: every access below names its slot statically, so the
  // compiler can tell the prefetch into one slot from the reads of another and does not make
  // those reads wait for the prefetch.  4-wave workgroups use four slots: two stages of two
  // key blocks each, one barrier per two blocks, the next pair prefetched while the current
  // one is computed (the 1-wave workgroups keep two slots: their LDS bounds occupancy).
  constexpr int XS = NW == 4 ? 1 : 0;   // slots 2 and 3 exist
  __shared__ __attribute__((aligned(16))) uint16_t sK0[KLOADS * 64 * 8], sK1[KLOADS * 64 * 8];
  __shared__ __attribute__((aligned(16))) uint32_t sV0[VROWS * VDW], sV1[VROWS * VDW];
  __shared__ __attribute__((aligned(16))) uint16_t sK2[XS * KLOADS * 64 * 8 + 8], sK3[XS * KLOADS * 64 * 8 + 8];
  __shared__ __attribute__((aligned(16))) uint32_t sV2[XS * VROWS * VDW + 4], sV3[XS * VROWS * VDW + 4];

  // ---- work unit: XCD-contiguous ranges of (head, unit), units of a segment adjacent
  if (DYN) n_work = *n_work_dev;
  const int G = n_work * a.heads;
  const int pid = blockIdx.x;
  if (pid >= G) return;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + local;
  const int head = logical / n_work;
  const AttnWork wk = work[logical % n_work];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int seg0 = wk.seg_start, n = wk.seg_len;
  const int qbase = wk.q0 + wv * 64;
  const uint16_t* Qh = a.q + (int64_t)head * a.n_tok * HD;
  const uint16_t* Kh = a.k + (int64_t)head * a.n_tok * HD;
  const uint16_t* Vh = a.vt + (int64_t)head * HD * a.vt_ld;

  // constant V^T rows: HD = ones (softmax denominator), the rest zeros; never overwritten
  for (int i = tid; i < (VROWS - HD) * VDW; i += NW * 64) {
    const uint32_t one2 = F16 ? 0x3c003c00u : 0x3f803f80u;   // pairs of 1.0 (float16 or bfloat16)
    const uint32_t v = i < VDW ? one2 : 0u;
    sV0[HD * VDW + i] = v;
    sV1[HD * VDW + i] = v;
    if (XS) {
      sV2[HD * VDW + i] = v;
      sV3[HD * VDW + i] = v;
    }
  }

  // ---- this wave's query fragments (B operand of S^T = K Q^T): query 32t + l32, dims 16c + 8h
  bf16x8 qf[QT][NCH];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int q = qbase + 32 * t + l32;
    const bool ok = q < n;
    const uint16_t* qr = Qh + (int64_t)(seg0 + (ok ? q : 0)) * HD + 8 * h;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
      qf[t][c] = ok ? v : bf16x8{};
    }
  }

  f32x16 O[QT][DT];
  float m[QT];
  f32x16 nm[QT];   // -m[t] in every entry: the score MFMAs start from it, so they yield s - m
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m[t] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) nm[t][e] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) O[t][dt][e] = 0.f;
  }
  // keys of this unit: with PART, blocks [kb0, kb1) of the segment (rows kseg..), kn of them
  // valid; the loop below runs over the unit's blocks 0.. either way
  const int kseg = PART ? seg0 + wk.kb0 * KB : seg0;
  const int kn = PART ? min(n, wk.kb1 * KB) - wk.kb0 * KB : n;
  const int nkb = (kn + KB - 1) / KB;

  // Direct global -> LDS tile loads through buffer resources over this head's K and V^T:
  // each lane keeps one 32-bit offset per load and the block's key offset rides in the
  // scalar offset.  The buffer range check covers the lane offset only, not the scalar one,
  // so reads past a segment's end are kept in bounds by the layout instead: K rows past the
  // end are the next segment's (or, for the last head, the V^T region that follows K), and
  // their scores are masked to -inf; a V^T row has at least 40 zeroed columns past the last
  // token (the planner's pitch), which covers the farthest read (31 tokens past a segment),
  // so the keys that get P = 0 multiply finite zeros, never stale memory.
  constexpr int KLW = (KLOADS + NW - 1) / NW, VLW = (VLOADS + NW - 1) / NW;
  const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kh), (short)0,
                                                    (int)(a.n_tok * HD * 2), kRsrcWord3);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vh), (short)0,
                                                    (int)(a.vt_ld * HD * 2), kRsrcWord3);
  // (fixed-size arrays: a dependent bound here fails the host-side instantiation with this
  // clang; only the first KLW / VLW entries are used)
  static_assert(KLW <= 8 && VLW <= 24, "load plan");
  uint32_t koff[8], voff[24];
#pragma unroll
  for (int j = 0; j < KLW; ++j) {
    const int id = (wv + j * NW) * 64 + lane, r = id / KCH, c = id % KCH;
    koff[j] = (uint32_t)(key_at(r) * HD + (c < HD / 8 ? c * 8 : 0)) * 2;
  }
#pragma unroll
  for (int j = 0; j < VLW; ++j) {
    const int id = (wv + j * NW) * 64 + lane, dd = id / VCH, q = id % VCH;
    const int c = q ^ ((dd >> 2) & 3);   // the global chunk that lands in slot q of row dd
    voff[j] = dd < HD ? (uint32_t)(dd * a.vt_ld + 8 * c) * 2 : 0u;
  }
  auto dload = [&](int kb, uint16_t* dK, uint32_t* dV) {
    const uint32_t key0 = (uint32_t)(kseg + kb * KB);
#pragma unroll
    for (int j = 0; j < KLW; ++j) {
      const int i = wv + j * NW;
      if (i >= KLOADS) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dK + i * 64 * 8), 16,
                                               koff[j], key0 * HD * 2, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < VLW; ++j) {
      const int i = wv + j * NW;
      if (i >= VLOADS) break;
      if (i * 64 + lane < HD * VCH)   // lanes past the real rows must not touch the constant rows
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(dV + i * 64 * 4), 16,
                                                 voff[j], key0 * 2, 0, 0);
    }
  };

  // one key block computed on (cK, cV); with sync, block kb + 1 is first prefetched into
  // (nK, nV) and the workgroup meets at a barrier after the block (the two-slot ring)
  auto block = [&](int kb, const uint16_t* cK, const uint32_t* cV, uint16_t* nK, uint32_t* nV, bool sync = true) {
    if (sync && kb + 1 < nkb) dload(kb + 1, nK, nV);
    if (qbase < n) {
      const uint16_t* Kt = cK;
      const uint16_t* Vt = reinterpret_cast<const uint16_t*>(cV);
      // ---- S^T = K Q^T for both query tiles: rows = 32 keys, columns = 32 queries
      f32x16 S[QT];
      const uint16_t* kr = Kt + l32 * KS + 8 * h;
      // K fragments three reads ahead of their MFMAs (the compiler's own order keeps two in
      // flight, so each pair of MFMAs would wait for its read)
      constexpr int KAH = NCH < 3 ? NCH : 3;
      bf16x8 kf[NCH];
#pragma unroll
      for (int c = 0; c < KAH; ++c) kf[c] = *reinterpret_cast<const bf16x8*>(kr + 16 * c);
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int t = 0; t < QT; ++t)
          S[t] = mma<F16>(kf[c], qf[t][c], c == 0 ? nm[t] : S[t]);
        if (c + KAH < NCH) kf[c + KAH] = *reinterpret_cast<const bf16x8*>(kr + 16 * (c + KAH));
      }
      __builtin_amdgcn_sched_group_barrier(0x100, KAH, 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, QT, 1);
        if (c + KAH < NCH) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      // ---- mask keys past the segment end (last step only); lane's keys are 8g + 4h + e
      const int key_base = kb * KB;
      if (key_base + KB > kn) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (key_base + key_at(8 * (e / 4) + 4 * h + (e % 4)) >= kn)
#pragma unroll
            for (int t = 0; t < QT; ++t) S[t][e] = -INFINITY;
      }
      // ---- online softmax per query (lazy offset: raised only by > 2^8)
      bf16x8 pb[QT][2];
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        // S holds s - m (s = q.k in log2 units: q carries log2(e) / sqrt(head_dim))
        float mx = S[t][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[t][e]);
        mx = max_xor32(mx);
        const bool need = kb == 0 || mx > 8.0f;
        if (__builtin_amdgcn_ballot_w64(need)) {
          // raise the offset by the block max where needed (always on the first block)
          const float mn = need ? m[t] + mx : m[t];
          const float dm = mn - m[t];
          if (kb > 0) {
            const float alpha = __builtin_amdgcn_exp2f(-dm);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) O[t][dt] *= alpha;
          }
          m[t] = mn;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            nm[t][e] = -mn;
            S[t][e] -= dm;
          }
        }
        if (t == QT - 1) __builtin_amdgcn_s_setprio(0);   // raised since the score MFMAs
        uint32_t pw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pw[i] = pack16<F16>(__builtin_amdgcn_exp2f(S[t][2 * i]), __builtin_amdgcn_exp2f(S[t][2 * i + 1]));
        pb[t][0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        pb[t][1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
      }
      // ---- O^T += V^T P^T over the 32 keys; the lane's probabilities of chunk c are the keys
      //      16c + 8h + 0..7 (K rows are loaded in key_at order), i.e. one whole 16-byte chunk
      //      2c + h of a V^T row
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int row = 32 * dt + l32;
        const uint16_t* vr = Vt + row * VP;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vr + 8 * ((2 * c + h) ^ ((row >> 2) & 3)));
#pragma unroll
          for (int t = 0; t < QT; ++t) O[t][dt] = mma<F16>(vf, pb[t][c], O[t][dt]);
        }
      }
    }
    if (sync) __syncthreads();
  };

  if constexpr (XS) {
    // two key blocks per barrier: slots (0, 2) hold one pair, (1, 3) the next; the barrier
    // after a pair makes the prefetched pair visible and frees the pair just read
    dload(0, sK0, sV0);
    if (1 < nkb) dload(1, sK2, sV2);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 4) {
      if (kb + 2 < nkb) dload(kb + 2, sK1, sV1);
      if (kb + 3 < nkb) dload(kb + 3, sK3, sV3);
      block(kb, sK0, sV0, nullptr, nullptr, false);
      if (kb + 1 < nkb) block(kb + 1, sK2, sV2, nullptr, nullptr, false);
      __syncthreads();
      if (kb + 2 >= nkb) break;
      if (kb + 4 < nkb) dload(kb + 4, sK0, sV0);
      if (kb + 5 < nkb) dload(kb + 5, sK2, sV2);
      block(kb + 2, sK1, sV1, nullptr, nullptr, false);
      if (kb + 3 < nkb) block(kb + 3, sK3, sV3, nullptr, nullptr, false);
      __syncthreads();
    }
  } else {
    dload(0, sK0, sV0);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
      block(kb, sK0, sV0, sK1, sV1);
      if (kb + 1 < nkb) block(kb + 1, sK1, sV1, sK0, sV0);
    }
  }

  if (qbase >= n) return;
  if (PART && wk.part >= 0) {
    // part of the query block's keys: the unnormalised output, the running offset and the
    // denominator go to the partial slot (rows of 256 queries, coalesced over the lanes)
    float* pb = a.part + ((int64_t)head * a.n_parts + wk.part) * (HD + 2) * 256;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int q = qbase + 32 * t + l32;
      if (q >= n) continue;
      const int qr = q - wk.q0;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int d = 32 * dt + 8 * (e / 4) + 4 * h + (e % 4);
          if (d < HD) pb[d * 256 + qr] = O[t][dt][e];
        }
      if (h == LHALF) pb[(HD + 1) * 256 + qr] = O[t][DT - 1][LIDX];
      if (h == 0) pb[HD * 256 + qr] = m[t];
    }
    return;
  }
  const int hid = a.heads * HD;
  const int ld = a.o_split ? 2 * hid : hid;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int q = qbase + 32 * t + l32;
    // the row sum sits in the lanes of one half: bring it to both halves
    const float lsum_own = O[t][DT - 1][LIDX];
    const float lsum = LHALF == 0 ? from_lower_half(lsum_own) : from_upper_half(lsum_own);
    if (q < n) {
      const float inv = 1.0f / lsum;
      // output row in the blocked GEMM layout (the out-projection's A operand); 4 values per
      // store, plus what their bf16 rounding leaves out when the out-projection compensates it
      const int64_t orow = seg0 + q;
      const int ocol = head * HD + 4 * h;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g;   // + 4h + e
          if (d + 8 > HD) continue;
          const f32x16& o = O[t][dt];
          const float y0 = o[4 * g] * inv, y1 = o[4 * g + 1] * inv, y2 = o[4 * g + 2] * inv,
                      y3 = o[4 * g + 3] * inv;
          *reinterpret_cast<uint2*>(a.o + kt_index(orow, ocol + d, ld)) =
              make_uint2(pack16<F16>(y0, y1), pack16<F16>(y2, y3));
          if (F16) continue;   // float16 output needs no compensation
          if (a.o_split)
            *reinterpret_cast<uint2*>(a.o + kt_index(orow, hid + ocol + d, ld)) =
                make_uint2(pack_bf16(bf16_rest(y0), bf16_rest(y1)), pack_bf16(bf16_rest(y2), bf16_rest(y3)));
          if (a.o8)
            *reinterpret_cast<uint32_t*>(a.o8 + kt8_index(orow, ocol + d, hid)) = rest_e4m3x4(y0, y1, y2, y3);
        }
    }
  }
}

template <int HD, bool F16>
hipError_t run_hd(const AttnArgs& a, hipStream_t st) {
  // key-split lists (partial slots given) take the PART instantiation; bucketed graphs (DYN)
  // run plain lists only
  if (a.n_long > 0 && a.n_long_dev)
    hipLaunchKernelGGL((attn_kernel<HD, 4, true, F16, false>), dim3(a.n_long * a.heads), dim3(256), 0, st, a,
                       a.work_long, a.n_long, a.n_long_dev);
  else if (a.n_long > 0 && a.part)
    hipLaunchKernelGGL((attn_kernel<HD, 4, false, F16, true>), dim3(a.n_long * a.heads), dim3(256), 0, st, a,
                       a.work_long, a.n_long, nullptr);
  else if (a.n_long > 0)
    hipLaunchKernelGGL((attn_kernel<HD, 4, false, F16, false>), dim3(a.n_long * a.heads), dim3(256), 0, st, a,
                       a.work_long, a.n_long, nullptr);
  if (a.n_short > 0 && a.n_short_dev)
    hipLaunchKernelGGL((attn_kernel<HD, 1, true, F16, false>), dim3(a.n_short * a.heads), dim3(64), 0, st, a,
                       a.work_short, a.n_short, a.n_short_dev);
  else if (a.n_short > 0)
    hipLaunchKernelGGL((attn_kernel<HD, 1, false, F16, false>), dim3(a.n_short * a.heads), dim3(64), 0, st, a,
                       a.work_short, a.n_short, nullptr);
  return hipGetLastError();
}

// Merge of key-split units: workgroup = (merge, head, 16 head dims), thread = query of the
// merge's 256-query block.  With the parts' running offsets m_p (log2 units) and M = max m_p,
// the output is sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p -- the rescale the attention
// kernel applies between key blocks, applied between parts.
template <int HD, bool F16>
__global__ void __launch_bounds__(256)
attn_merge_kernel(AttnArgs a, const AttnMerge* __restrict__ merges) {
  constexpr int DG = HD / 16;          // groups of 16 head dims
  constexpr int PS = (HD + 2) * 256;   // floats per partial slot
  const int dg = blockIdx.x % DG, head = (blockIdx.x / DG) % a.heads;
  const AttnMerge mg = merges[blockIdx.x / DG / a.heads];
  const int qr = threadIdx.x, q = mg.q0 + qr;
  if (q >= mg.seg_len) return;
  const float* pb = a.part + ((int64_t)head * a.n_parts + mg.part0) * PS + qr;
  const int np = mg.n_parts;
  float mx = -INFINITY;
  for (int p = 0; p < np; ++p) mx = fmaxf(mx, pb[p * PS + HD * 256]);
  float l = 0.f, y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) y[j] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float* pp = pb + p * PS;
    const float w = __builtin_amdgcn_exp2f(pp[HD * 256] - mx);
    l += w * pp[(HD + 1) * 256];
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] += w * pp[(16 * dg + j) * 256];
  }
  const float inv = 1.0f / l;
  const int64_t orow = mg.seg_start + q;
#pragma unroll
  for (int j = 0; j < 16; j += 4)
    store_o4<F16>(a, orow, head * HD + 16 * dg + j, y[j] * inv, y[j + 1] * inv, y[j + 2] * inv, y[j + 3] * inv);
}

// Zeroes V^T columns [n, n + 64) (clipped to the pitch) of every row: the attention's tile
// loads read at most 31 keys past the last token, and the pitch leaves at least 40 columns.  n is the token count, read at run time
// when n_tok_dev is set (bucketed graph).
__global__ void vt_pad_zero_kernel(uint16_t* vt, int rows, int64_t n_tok, const int32_t* n_tok_dev, int64_t vt_ld) {
  const int64_t n = n_tok_dev ? (int64_t)*n_tok_dev : n_tok;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * 64) return;
  const int64_t col = n + (i & 63);
  if (col < vt_ld) vt[(i >> 6) * vt_ld + col] = 0;
}

}  // namespace

vit_status launch_vt_pad_zero(uint16_t* vt, int rows, int64_t n_tok, int64_t vt_ld, void* stream,
                              const int32_t* n_tok_dev) {
  if ((vt_ld <= n_tok && !n_tok_dev) || rows <= 0) return VIT_OK;
  const int64_t n = (int64_t)rows * 64;
  hipLaunchKernelGGL(vt_pad_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), vt, rows, n_tok, n_tok_dev, vt_ld);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("V^T pad clear: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

vit_status launch_attention_merge(const AttnArgs& a, const AttnMerge* merge, int n_merge, void* stream) {
  if (n_merge <= 0) return VIT_OK;
  if (!a.part || a.n_parts <= 0 || !merge) {
    set_error("attention merge: no partial slots");
    return VIT_E_ARG;
  }
  if (a.f16 && (a.o_split || a.o8)) {
    set_error("attention merge: float16 output takes no compensation");
    return VIT_E_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(n_merge * a.heads * (a.head_dim / 16)));
  switch (a.head_dim) {
    case 32:
      if (a.f16) hipLaunchKernelGGL((attn_merge_kernel<32, true>), grid, dim3(256), 0, st, a, merge);
      else hipLaunchKernelGGL((attn_merge_kernel<32, false>), grid, dim3(256), 0, st, a, merge);
      break;
    case 64:
      if (a.f16) hipLaunchKernelGGL((attn_merge_kernel<64, true>), grid, dim3(256), 0, st, a, merge);
      else hipLaunchKernelGGL((attn_merge_kernel<64, false>), grid, dim3(256), 0, st, a, merge);
      break;
    case 80:
      if (a.f16) hipLaunchKernelGGL((attn_merge_kernel<80, true>), grid, dim3(256), 0, st, a, merge);
      else hipLaunchKernelGGL((attn_merge_kernel<80, false>), grid, dim3(256), 0, st, a, merge);
      break;
    default:
      set_error("attention merge: head_dim %d not supported (32, 64, 80)", a.head_dim);
      return VIT_E_ARG;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention merge launch: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  return VIT_OK;
}

vit_status launch_attention(const AttnArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.vt_ld < a.n_tok + 40 || a.vt_ld % 8) {
    set_error("attention: V^T pitch %lld must be a multiple of 8 and cover %lld tokens plus 40 pad columns",
              (long long)a.vt_ld, (long long)a.n_tok);
    return VIT_E_ARG;
  }
  if (a.vt_ld * a.head_dim * 2 >= ((int64_t)1 << 31)) {
    set_error("attention: %lld tokens exceed the 2 GiB per-head operand limit", (long long)a.n_tok);
    return VIT_E_ARG;
  }
  hipError_t e;
  if (a.f16 && (a.o_split || a.o8)) {
    set_error("attention: float16 output takes no compensation");
    return VIT_E_ARG;
  }
  switch (a.head_dim) {
    case 32: e = a.f16 ? run_hd<32, true>(a, st) : run_hd<32, false>(a, st); break;
    case 64: e = a.f16 ? run_hd<64, true>(a, st) : run_hd<64, false>(a, st); break;
    case 80: e = a.f16 ? run_hd<80, true>(a, st) : run_hd<80, false>(a, st); break;
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
