// Exp-kernel contractions of WildCat on gfx950 matrix cores.
//
//   weights (CompressKV):  Y[a, :] = sum_b exp(c <k_a, k_b> + rowc_a + colc_b) [V_b, 1]
//   attend  (WtdAttn):     N[i, :] = sum_j exp(beta <q_i, ks_j>) X_j,  O = clip(N[:, :d] / N[:, d])
//
// [WildCat (arXiv 2602.10056): plug-in estimator paragraph (W [V, 1] is formed
// before the queries are applied), Lem. 1 paragraph (clip to the column value
// range), CompressKV / Alg. 2 and WtdAttn / Alg. 3 paragraphs.]
//
// bf16 inputs with d >= 32 run expmm32 (32x32x16 MFMA, described at the
// kernel); d = 16 runs expmm_bf16, and fp32 inputs run expmm_f32m on the
// fp32 matrix cores (described at the kernel).  expmm_bf16: a workgroup of NW waves owns 16 rows of the
// left operand per wave (fragments kept in registers) and streams the right
// operand in tiles of 64 rows through LDS.  Per 32 right rows a wave issues
//   scores^T (16 rows x 16 cols) x2 : v_mfma_f32_16x16x32_bf16 over d
//   P = exp2(...) in fp32, rounded to bf16 in registers
//   P x [V] (16 x d)                : v_mfma_f32_16x16x32_bf16 over the 32 rows
// The score tiles are computed transposed with a row permutation chosen so
// that every lane ends up holding 8 consecutive right rows of its own left row,
// which is exactly the A-operand layout of the second MFMA: P never leaves the
// registers.  V is staged transposed in LDS so the second MFMA's B operand is
// one 16-byte LDS read.  The last column ([.., 1] or w) is accumulated on the
// vector ALU (expmm_bf16: from the bf16-rounded P; expmm32: from P in fp32
// before rounding).  No running maximum is needed: the exponents are bounded
// by the input-range contract.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "keymean.hpp"
#include "ordered.hpp"
#include "weights_layout.hpp"

namespace wc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct ContractArgs {
  const void* A;        // left rows  [units][rowsA][D] (bf16 or fp32)
  const void* B;        // right rows [unitsB][rowsB][D]
  const void* Vs;       // values: V [unitsB][rowsB][D] (weights) or X [unitsB][rowsB][D+1] fp32 (attend)
  const float* rowc;    // [units][rowsA] exponent offsets (weights + recentring) or null
  const float* colc;    // [unitsB][rowsB] exponent offsets (weights + recentring) or null
  float* out;           // weights: ypart [nsplit][units][rowsA][D+1]; attend: O [units][rowsA][D]
  const float* vmin;    // attend: [unitsB][D], or [unitsB][rowsA][D] with range_rows
  const float* vmax;
  int rowsA, rowsB;
  int chunk;            // right rows per split (weights); rowsB for attend
  int group;            // left unit u reads right unit u / group (GQA); 1 for weights
  int units;
  float scale;          // c (weights) or beta (attend)
  // Attend over a cache with appended tokens: with `causal`, right row b >=
  // causal_from is seen by left row a only when b - causal_from <= a.
  int causal, causal_from;
  int range_rows;       // attend: clip range per left row instead of per unit
};

// Right row b is visible to left row a (attend over a cache with appended tokens).
__device__ __forceinline__ bool visible(const ContractArgs& p, int b, int a) {
  return !p.causal || b - p.causal_from <= a;
}

enum { kModeWeights = 0, kModeAttend = 1 };

// Physical LDS row of right row `k` inside its 32-row block: the rows one
// score MFMA reads (lanes 0..15) become 16 consecutive LDS rows.
__device__ __forceinline__ int perm_row(int k) {
  const int blk = k & ~31, w = k & 31;
  const int a = w >> 3, t = (w >> 2) & 1, i = w & 3;
  return blk + 16 * t + 4 * a + i;
}

template <int D, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void expmm_bf16(ContractArgs p) {
  constexpr int NTH = 64 * NW;       // threads; the workgroup owns 16 * NW left rows
  constexpr int KP = D + 8;          // LDS row pitch of the right tile (bf16)
  constexpr int VP = kTileKeys + 8;  // LDS row pitch of the transposed values (bf16)
  constexpr int DK = D < 32 ? 1 : D / 32;
  constexpr int CT = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sB[kTileKeys * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sVT[D * VP];
  __shared__ float sE[kTileKeys];
  __shared__ float sC[kTileKeys];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int unit = blockIdx.z;
  const int unitB = unit / p.group;
  const int a0 = blockIdx.y * 16 * NW;
  const int split = blockIdx.x;
  const int b_begin = MODE == kModeWeights ? split * p.chunk : 0;
  int b_end = MODE == kModeWeights ? min(p.rowsB, b_begin + p.chunk) : p.rowsB;
  // causal: right rows hidden from every left row of the workgroup are skipped
  if (MODE == kModeAttend && p.causal) b_end = min(b_end, p.causal_from + a0 + 16 * NW);

  const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + (size_t)unit * p.rowsA * D;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + (size_t)unitB * p.rowsB * D;

  // Left-row fragments: lane holds row a0 + 16*wave + r16, k = 32*dk + 8*g .. +7.
  const int arow = a0 + wave * 16 + r16;
  bf16x8 afrag[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    const int k0 = 32 * dk + 8 * g;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (arow < p.rowsA && k0 < D) v = *reinterpret_cast<const uint4*>(A + (size_t)arow * D + k0);
    afrag[dk] = __builtin_bit_cast(bf16x8, v);
  }
  float rc2 = 0.0f;
  if (MODE == kModeWeights && p.rowc != nullptr && arow < p.rowsA) rc2 = p.rowc[(size_t)unit * p.rowsA + arow] * kLog2e;
  const float sc2 = p.scale * kLog2e;

  f32x4 oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float eacc = 0.0f;

  for (int b0 = b_begin; b0 < b_end; b0 += kTileKeys) {
    // ---- stage the right tile (permuted rows) and the transposed values
    for (int q = t; q < kTileKeys * (D / 8); q += NTH) {
      const int row = q / (D / 8), c8 = q % (D / 8);
      const int b = b0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (b < b_end) v = *reinterpret_cast<const uint4*>(B + (size_t)b * D + 8 * c8);
      *reinterpret_cast<uint4*>(&sB[perm_row(row) * KP + 8 * c8]) = v;
    }
    for (int q = t; q < (kTileKeys / 2) * (D / 8); q += NTH) {
      const int rp = q % (kTileKeys / 2), c8 = q / (kTileKeys / 2);
      const int b = b0 + 2 * rp;
      uint32_t lo[8], hi[8];
      if (MODE == kModeWeights) {
        const uint16_t* V = reinterpret_cast<const uint16_t*>(p.Vs) + (size_t)unitB * p.rowsB * D;
        uint4 x = make_uint4(0u, 0u, 0u, 0u), y = make_uint4(0u, 0u, 0u, 0u);
        if (b < b_end) x = *reinterpret_cast<const uint4*>(V + (size_t)b * D + 8 * c8);
        if (b + 1 < b_end) y = *reinterpret_cast<const uint4*>(V + (size_t)(b + 1) * D + 8 * c8);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[2 * j] = xs[j] & 0xFFFFu; lo[2 * j + 1] = xs[j] >> 16;
          hi[2 * j] = ys[j] & 0xFFFFu; hi[2 * j + 1] = ys[j] >> 16;
        }
      } else {
        const float* X = reinterpret_cast<const float*>(p.Vs) + (size_t)unitB * p.rowsB * (D + 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = b < b_end ? X[(size_t)b * (D + 1) + 8 * c8 + j] : 0.0f;
          const float y = b + 1 < b_end ? X[(size_t)(b + 1) * (D + 1) + 8 * c8 + j] : 0.0f;
          lo[j] = __builtin_bit_cast(uint16_t, (__bf16)x);
          hi[j] = __builtin_bit_cast(uint16_t, (__bf16)y);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint32_t*>(&sVT[(8 * c8 + j) * VP + 2 * rp]) = lo[j] | (hi[j] << 16);
    }
    for (int q = t; q < kTileKeys; q += NTH) {
      const int b = b0 + q;
      if (MODE == kModeAttend) {
        const float* X = reinterpret_cast<const float*>(p.Vs) + (size_t)unitB * p.rowsB * (D + 1);
        sE[q] = b < b_end ? X[(size_t)b * (D + 1) + D] : 0.0f;
      } else {
        sE[q] = b < b_end ? 1.0f : 0.0f;
        sC[q] = (p.colc != nullptr && b < b_end) ? p.colc[(size_t)unitB * p.rowsB + b] * kLog2e : 0.0f;
      }
    }
    __syncthreads();

    // ---- two 32-row blocks per tile
#pragma unroll
    for (int kb = 0; kb < kTileKeys / 32; ++kb) {
      float pv[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
          const int k0 = 32 * dk + 8 * g;
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (k0 < D) v = *reinterpret_cast<const uint4*>(&sB[(32 * kb + 16 * tt + r16) * KP + k0]);
          s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), afrag[dk], s4, 0, 0, 0);
        }
        // s4[i] = score of left row r16 with right row 32kb + 8g + 4tt + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = 32 * kb + 8 * g + 4 * tt + i;
          float arg = fmaf(s4[i], sc2, rc2);
          if (MODE == kModeWeights) arg += sC[kk];
          pv[4 * tt + i] = sE[kk] != 0.0f || MODE == kModeAttend ? exp2f(arg) : 0.0f;
        }
      }
      // bf16 P as the A operand of the value MFMA; extra column on the VALU.
      // Attend: right rows past rowsB (staged as zeros) and rows hidden by
      // the causal mask get P = 0.
      bf16x8 pfrag;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = 32 * kb + 8 * g + j;
        const bool keep = MODE != kModeAttend || (b0 + kk < b_end && visible(p, b0 + kk, arow));
        const __bf16 h = keep ? (__bf16)pv[j] : (__bf16)0.0f;
        pfrag[j] = h;
        eacc = fmaf((float)h, sE[kk], eacc);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sVT[(16 * ct + r16) * VP + 32 * kb + 8 * g]);
        oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pfrag, __builtin_bit_cast(bf16x8, v), oacc[ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // eacc: partial over this lane's 8-row groups -> full sum for left row r16.
  eacc += __shfl_xor(eacc, 16, 64);
  eacc += __shfl_xor(eacc, 32, 64);

  // oacc[ct][i] = result for left row 16*wave + 4g + i, column 16ct + r16.
  if (MODE == kModeWeights) {
    float* Y = p.out + ((size_t)split * p.units + unit) * p.rowsA * (D + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = a0 + wave * 16 + 4 * g + i;
      if (row < p.rowsA) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Y[(size_t)row * (D + 1) + 16 * ct + r16] = oacc[ct][i];
      }
    }
    if (g == 0 && arow < p.rowsA) Y[(size_t)arow * (D + 1) + D] = eacc;
  } else {
    float* O = p.out + (size_t)unit * p.rowsA * D;
    float lo[CT], hi[CT];   // read once: O stores could alias them
    if (!p.range_rows) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        lo[ct] = p.vmin[(size_t)unitB * D + 16 * ct + r16];
        hi[ct] = p.vmax[(size_t)unitB * D + 16 * ct + r16];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 4 * g + i;
      const float e = __shfl(eacc, rl, 64);
      const int row = a0 + wave * 16 + rl;
      if (row < p.rowsA) {
        if (p.range_rows) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const size_t k = ((size_t)unitB * p.rowsA + row) * D + 16 * ct + r16;
            lo[ct] = p.vmin[k];
            hi[ct] = p.vmax[k];
          }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const float x = oacc[ct][i] / e;
          O[(size_t)row * D + 16 * ct + r16] = fminf(fmaxf(x, lo[ct]), hi[ct]);
        }
      }
    }
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Physical LDS row of key k inside its 32-key block for the 32x32 kernel:
// bits 2 and 3 of the index swapped (an involution).  With this placement the
// 32x32x16 score MFMA leaves, in every lane, the probabilities of its own left
// row for 8 consecutive keys per 16-key block -- the A-operand layout of the
// value MFMA.
__device__ __forceinline__ int perm32(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Same contraction with v_mfma_f32_32x32x16_bf16: each wave owns 32 left rows.
// KS = 1: NWAVE waves share double-buffered LDS tiles of KT right rows
// (loaded into registers one tile ahead, one barrier per tile; KT = 16 NWAVE,
// so the 8-wave configuration uses 139 KiB of the 160 KiB LDS and one tile of
// MFMA work covers the next tile's load latency).  KS > 1 (attend with few
// query rows): the right rows are split into KS contiguous ranges, each taken
// by RW = NWAVE / KS waves (RW row blocks) that stage their own 32-row tiles
// in a private LDS region.  With RW = 1 the region is single-buffered and
// the loop has no barrier (a wave's LDS accesses execute in order); with
// RW = 2 it is double-buffered as for KS = 1 (all ranges run the same number
// of tiles, so the barrier is shared).  The KS partial sums meet in LDS and
// are added in a fixed order.  Per 32 right rows a wave issues D/16 score
// MFMAs and 2*D/32 value MFMAs.  d >= 32.
#ifndef WILDCAT_MFMA32_KTMAX
#define WILDCAT_MFMA32_KTMAX 128
#endif
#ifndef WILDCAT_MFMA32_SCHEDBAR
#define WILDCAT_MFMA32_SCHEDBAR 0   // scheduling barrier before staging also in the shared-tile form
#endif
template <int D, int MODE, int NWAVE, bool RC, int KS>
struct Mfma32Cfg {
  static constexpr int RW = NWAVE / KS;                 // waves sharing one tile (same right rows)
  static_assert(RW * KS == NWAVE, "waves = row blocks x key ranges");
  static constexpr int NTH = 64 * RW;                   // threads staging one tile
  static constexpr int KT = KS > 1 ? 32 : ((16 * NWAVE < WILDCAT_MFMA32_KTMAX) ? 16 * NWAVE : WILDCAT_MFMA32_KTMAX);
  static constexpr int NBUF = (KS > 1 && RW == 1) ? 1 : 2;
  static constexpr int KP = D + 8;                      // bf16 pitch of a right row in LDS
  static constexpr int VP = KT + 8;                     // bf16 pitch of a transposed value row
  static constexpr int CT = D / 32;
  static constexpr size_t B_BYTES = (size_t)KT * KP * 2, VT_BYTES = (size_t)D * VP * 2, E_BYTES = (size_t)KT * 4;
  static constexpr size_t BUF_BYTES = B_BYTES + VT_BYTES + 2 * E_BYTES;   // keys, values^T, w, offsets
  static constexpr size_t TILE_BYTES = (size_t)KS * NBUF * BUF_BYTES;
  static constexpr size_t RED_BYTES = KS > 1 ? (size_t)NWAVE * 64 * (16 * CT + 1) * 4 : 0;
  static constexpr size_t LDS_BYTES = TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES;
};

template <int D, int MODE, int NWAVE, bool RC, int KS>
__global__ __launch_bounds__(64 * NWAVE) void expmm32(ContractArgs p) {
  using Cfg = Mfma32Cfg<D, MODE, NWAVE, RC, KS>;
  constexpr int NTH = Cfg::NTH, KT = Cfg::KT, KP = Cfg::KP, VP = Cfg::VP, CT = Cfg::CT;
  constexpr int DK = D / 16;
  constexpr int KI = KT * (D / 8);         // 16-byte right-row items per tile
  // Value items: weights (bf16 V) (row pair, 8 columns), one 16-byte load per
  // row; attend (fp32 X, rows of d + 1 values: 4-byte aligned only) (row
  // pair, 4 columns), one 16-byte load per row (global memory takes 16-byte
  // loads at 4-byte alignment), the 64 items of a wave spanning 8 row pairs
  // x 8 column quads (8 rows of 128 contiguous bytes per load instruction,
  // at most 2-way bank conflicts on the transposed LDS stores).
  constexpr int VI = MODE == kModeWeights ? (KT / 2) * (D / 8) : (KT / 2) * (D / 4);
  static_assert(MODE == kModeWeights || (KT % 16 == 0 && D % 32 == 0), "attend value items: 8 x 8 blocks");
  auto xitem = [](int it, int& rp, int& c4) __attribute__((always_inline)) {
    const int blk = it >> 6, w = it & 63;
    rp = (w & 7) + 8 * (blk / (D / 32));
    c4 = (w >> 3) + 8 * (blk % (D / 32));
  };
  constexpr int KIPT = (KI + NTH - 1) / NTH;
  constexpr int VIPT = (VI + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];

  const int t = threadIdx.x, lane = t & 63, wave = KS > 1 ? __builtin_amdgcn_readfirstlane(t >> 6) : t >> 6;
  const int g2 = lane >> 5, r32 = lane & 31;
  const int rw = wave % Cfg::RW;                    // row block of the wave
  const int ks = wave / Cfg::RW;                    // key range of the wave
  const int gt = t - ks * NTH;                      // thread index among those staging one tile
  char* const my_lds = lds + (size_t)ks * Cfg::NBUF * Cfg::BUF_BYTES;
  auto sB = [&](int b) { return reinterpret_cast<uint16_t*>(my_lds + b * Cfg::BUF_BYTES); };
  auto sVT = [&](int b) { return reinterpret_cast<uint16_t*>(my_lds + b * Cfg::BUF_BYTES + Cfg::B_BYTES); };
  auto sE = [&](int b) { return reinterpret_cast<float*>(my_lds + b * Cfg::BUF_BYTES + Cfg::B_BYTES + Cfg::VT_BYTES); };
  auto sC = [&](int b) {
    return reinterpret_cast<float*>(my_lds + b * Cfg::BUF_BYTES + Cfg::B_BYTES + Cfg::VT_BYTES + Cfg::E_BYTES);
  };
  const int unit = blockIdx.z, unitB = unit / p.group;
  const int a0 = blockIdx.y * 32 * Cfg::RW;
  const int split = blockIdx.x;
  int b_begin = MODE == kModeWeights ? split * p.chunk : 0;
  int b_end = MODE == kModeWeights ? min(p.rowsB, b_begin + p.chunk) : p.rowsB;
  // causal: right rows hidden from every left row of the workgroup are
  // skipped (not in the key-split form, whose waves share a barrier count)
  if (KS == 1 && MODE == kModeAttend && p.causal) b_end = min(b_end, p.causal_from + a0 + 32 * Cfg::RW);
  int ntiles = (b_end - b_begin + KT - 1) / KT;
  if (KS > 1) {
    // Equal ranges of whole 32-row blocks; every wave runs the same number of
    // tiles (a range past the end is all masked).
    const int per = ((p.rowsB + KS - 1) / KS + KT - 1) / KT * KT;
    b_begin = ks * per;
    b_end = min(p.rowsB, b_begin + per);
    ntiles = per / KT;
  }
  const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + (size_t)unit * p.rowsA * D;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + (size_t)unitB * p.rowsB * D;

  // Left-row fragments (B operand of the score MFMA): row a0 + 32 wave + r32,
  // d = 16 dk + 8 g2 .. +7.
  const int arow = a0 + rw * 32 + r32;
  bf16x8 afrag[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (arow < p.rowsA) v = *reinterpret_cast<const uint4*>(A + (size_t)arow * D + 16 * dk + 8 * g2);
    afrag[dk] = __builtin_bit_cast(bf16x8, v);
  }
  float rc2 = 0.0f;
  if (MODE == kModeWeights && p.rowc != nullptr && arow < p.rowsA) rc2 = p.rowc[(size_t)unit * p.rowsA + arow] * kLog2e;
  const float sc2 = p.scale * kLog2e;

  // ---- tile staging through registers.  load_tile only issues loads into
  // registers; everything that consumes them (packing, LDS stores) happens in
  // store_tile after the compute, so the loads overlap one tile of MFMA work.
  // Prefetch registers as vector values (never stack arrays).
  typedef uint32_t kvec_t __attribute__((ext_vector_type(4 * KIPT)));
  typedef uint32_t vvec_t __attribute__((ext_vector_type(MODE == kModeWeights ? 8 * VIPT : 1)));
  typedef float xvec_t __attribute__((ext_vector_type(MODE == kModeAttend ? 8 * VIPT : 1)));
  typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
  kvec_t kreg = {};           // right-row tile: 16 bytes per item
  vvec_t vreg = {};           // weights: rows 2rp and 2rp+1, 8 bf16 columns each
  xvec_t xreg = {};           // attend: X[2rp][4c4 .. +3] and X[2rp+1][4c4 .. +3] in fp32
  float ereg = 0.0f, creg = 0.0f;
  // Rows past b_end are read from the last valid row instead (no branches
  // around the loads): their probabilities are masked to 0, so only
  // finiteness matters.
  auto load_tile = [&](int b0) __attribute__((always_inline)) {
    const int blast = max(min(b_end, p.rowsB) - 1, 0);
#pragma unroll
    for (int q = 0; q < KIPT; ++q) {
      const int it = gt + q * NTH;
      if (KI % NTH == 0 || it < KI) {
        const int row = it / (D / 8), c8 = it % (D / 8);
        const int b = min(b0 + row, blast);
        const uint4 x = *reinterpret_cast<const uint4*>(B + (size_t)b * D + 8 * c8);
        kreg[4 * q] = x.x; kreg[4 * q + 1] = x.y; kreg[4 * q + 2] = x.z; kreg[4 * q + 3] = x.w;
      }
    }
#pragma unroll
    for (int q = 0; q < VIPT; ++q) {
      const int it = gt + q * NTH;
      if (VI % NTH == 0 || it < VI) {
        if constexpr (MODE == kModeWeights) {
          const int rp = it % (KT / 2), c8 = it / (KT / 2);
          const int b = min(b0 + 2 * rp, blast), b1 = min(b0 + 2 * rp + 1, blast);
          const uint16_t* V = reinterpret_cast<const uint16_t*>(p.Vs) + (size_t)unitB * p.rowsB * D;
          const uint4 x = *reinterpret_cast<const uint4*>(V + (size_t)b * D + 8 * c8);
          const uint4 y = *reinterpret_cast<const uint4*>(V + (size_t)b1 * D + 8 * c8);
          vreg[8 * q] = x.x; vreg[8 * q + 1] = x.y; vreg[8 * q + 2] = x.z; vreg[8 * q + 3] = x.w;
          vreg[8 * q + 4] = y.x; vreg[8 * q + 5] = y.y; vreg[8 * q + 6] = y.z; vreg[8 * q + 7] = y.w;
        } else {
          const float* X = reinterpret_cast<const float*>(p.Vs) + (size_t)unitB * p.rowsB * (D + 1);
          int rp, c4;
          xitem(it, rp, c4);
          const int b = min(b0 + 2 * rp, blast), b1 = min(b0 + 2 * rp + 1, blast);
          const f4u x = *reinterpret_cast<const f4u*>(X + ((size_t)b * (D + 1) + 4 * c4));
          const f4u y = *reinterpret_cast<const f4u*>(X + ((size_t)b1 * (D + 1) + 4 * c4));
          xreg[8 * q] = x.x; xreg[8 * q + 1] = x.y; xreg[8 * q + 2] = x.z; xreg[8 * q + 3] = x.w;
          xreg[8 * q + 4] = y.x; xreg[8 * q + 5] = y.y; xreg[8 * q + 6] = y.z; xreg[8 * q + 7] = y.w;
        }
      }
    }
    if (gt < KT) {
      const int b = min(b0 + gt, blast);
      if (MODE == kModeAttend) {
        const float* X = reinterpret_cast<const float*>(p.Vs) + (size_t)unitB * p.rowsB * (D + 1);
        ereg = X[(size_t)b * (D + 1) + D];
      }
      if (RC) creg = p.colc[(size_t)unitB * p.rowsB + b];
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < KIPT; ++q) {
      const int it = gt + q * NTH;
      if (KI % NTH == 0 || it < KI) {
        const int row = it / (D / 8), c8 = it % (D / 8);
        *reinterpret_cast<uint4*>(&sB(buf)[perm32(row) * KP + 8 * c8]) =
            make_uint4(kreg[4 * q], kreg[4 * q + 1], kreg[4 * q + 2], kreg[4 * q + 3]);
      }
    }
#pragma unroll
    for (int q = 0; q < VIPT; ++q) {
      const int it = gt + q * NTH;
      if (VI % NTH == 0 || it < VI) {
        if constexpr (MODE == kModeWeights) {
          const int rp = it % (KT / 2), c8 = it / (KT / 2);
          uint32_t w[8];
          const uint32_t xs[4] = {vreg[8 * q], vreg[8 * q + 1], vreg[8 * q + 2], vreg[8 * q + 3]};
          const uint32_t ys[4] = {vreg[8 * q + 4], vreg[8 * q + 5], vreg[8 * q + 6], vreg[8 * q + 7]};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            w[2 * j] = (xs[j] & 0xFFFFu) | (ys[j] << 16);
            w[2 * j + 1] = (xs[j] >> 16) | (ys[j] & 0xFFFF0000u);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(&sVT(buf)[(8 * c8 + j) * VP + 2 * rp]) = w[j];
        } else {
          int rp, c4;
          xitem(it, rp, c4);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint32_t*>(&sVT(buf)[(4 * c4 + j) * VP + 2 * rp]) =
                (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)xreg[8 * q + j]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)xreg[8 * q + 4 + j]) << 16);
        }
      }
    }
    if (gt < KT) {
      if (MODE == kModeAttend) sE(buf)[gt] = ereg;
      if (RC) sC(buf)[gt] = creg * kLog2e;
    }
  };

  f32x16 oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[ct][v] = 0.0f;
  float eacc = 0.0f;

  // Scores of the wave's 32 left rows against right rows kofs .. kofs+31 of
  // the tile in buffer `bf`: s[v] = <left r32, right kofs + k(v)>,
  // k(v) = 16 (v/8) + 8 g2 + v % 8 (the perm32 placement).
  auto scores = [&](int bf, int kofs) __attribute__((always_inline)) {
    f32x16 acc = {};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const uint4 v = *reinterpret_cast<const uint4*>(&sB(bf)[(kofs + r32) * KP + 16 * dk + 8 * g2]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), afrag[dk], acc, 0, 0, 0);
    }
    return acc;
  };
  // Probabilities exp2(scale2 * s + offsets) as bf16 in the value MFMA's
  // A-operand layout, and the last-column sum from the fp32 values before
  // rounding (no conversion back from bf16 on the vector ALU).
  auto probs = [&](auto masked_tag, const f32x16& sv, int bf, int kofs, int b0, bf16x8 (&pfrag)[2]) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float ev[16], cv[16];
    if (MODE == kModeAttend) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 e0 = *reinterpret_cast<const float4*>(&sE(bf)[kofs + 16 * kb + 8 * g2]);
        const float4 e1 = *reinterpret_cast<const float4*>(&sE(bf)[kofs + 16 * kb + 8 * g2 + 4]);
        ev[8 * kb + 0] = e0.x; ev[8 * kb + 1] = e0.y; ev[8 * kb + 2] = e0.z; ev[8 * kb + 3] = e0.w;
        ev[8 * kb + 4] = e1.x; ev[8 * kb + 5] = e1.y; ev[8 * kb + 6] = e1.z; ev[8 * kb + 7] = e1.w;
      }
    }
    if (RC) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 c0 = *reinterpret_cast<const float4*>(&sC(bf)[kofs + 16 * kb + 8 * g2]);
        const float4 c1 = *reinterpret_cast<const float4*>(&sC(bf)[kofs + 16 * kb + 8 * g2 + 4]);
        cv[8 * kb + 0] = c0.x; cv[8 * kb + 1] = c0.y; cv[8 * kb + 2] = c0.z; cv[8 * kb + 3] = c0.w;
        cv[8 * kb + 4] = c1.x; cv[8 * kb + 5] = c1.y; cv[8 * kb + 6] = c1.z; cv[8 * kb + 7] = c1.w;
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float arg = fmaf(sv[v], sc2, rc2);
      if (RC) arg += cv[v];
      float pv = __builtin_amdgcn_exp2f(arg);
      if (MASKED) {
        const int b = b0 + kofs + 16 * (v >> 3) + 8 * g2 + (v & 7);
        pv = (b < b_end && (MODE != kModeAttend || visible(p, b, arow))) ? pv : 0.0f;
      }
      const __bf16 h = (__bf16)pv;
      pfrag[v >> 3][v & 7] = h;
      eacc = MODE == kModeAttend ? fmaf(pv, ev[v], eacc) : eacc + pv;
    }
  };
  // oacc += P (32 rows x 32 right rows) x V (32 right rows x D).
  auto values = [&](int bf, int kofs, const bf16x8 (&pfrag)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sVT(bf)[(32 * ct + r32) * VP + kofs + 16 * kb + 8 * g2]);
        oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pfrag[kb], __builtin_bit_cast(bf16x8, v), oacc[ct], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) {
    load_tile(b_begin);
    store_tile(0);
  }
  __syncthreads();
  int buf = 0;
  for (int it = 0; it < ntiles; ++it) {
    const int b0 = b_begin + it * KT;
    // Unconditional prefetch (the last tile re-loads itself into the idle
    // buffer): keeps the loads out of branches so they stay in flight.  An
    // attend over a single tile (few pivots, many query rows) has nothing to
    // prefetch and skips it, and the staging and barrier after it.
    const bool prefetch = MODE != kModeAttend || KS > 1 || ntiles > 1;
    const int bnext = it + 1 < ntiles ? b0 + KT : b0;
    if (prefetch) load_tile(bnext);

    // Software pipeline over the tile's 32-row blocks: the score MFMAs of
    // block k+1 are issued before the probabilities of block k are computed,
    // so the VALU work co-executes with the matrix core.
    // (Not in the key-split form: there the loads dominate and the second
    // score tile's registers are needed for the prefetch.)
    constexpr bool PIPE = KS == 1;
    f32x16 s_next = {};
    if (PIPE) s_next = scores(buf, 0);
    // A tile takes the masked path if it runs past b_end or holds a right
    // row that the causal mask hides from the wave's first left row.
    const bool full_tile = b0 + KT <= b_end && (MODE != kModeAttend || visible(p, b0 + KT - 1, a0 + rw * 32));
#pragma unroll
    for (int kb32 = 0; kb32 < KT / 32; ++kb32) {
      const f32x16 s_cur = PIPE ? s_next : scores(buf, 32 * kb32);
      if (PIPE && kb32 + 1 < KT / 32) s_next = scores(buf, 32 * (kb32 + 1));
      bf16x8 pfrag[2];
      if (full_tile) probs(std::false_type{}, s_cur, buf, 32 * kb32, b0, pfrag);
      else probs(std::true_type{}, s_cur, buf, 32 * kb32, b0, pfrag);
      values(buf, 32 * kb32, pfrag);
    }
    // Keep the staging of the next tile (which waits for its loads) after
    // this tile's MFMAs: without the barrier the scheduler interleaves the
    // two and every tile waits for its successor's loads.
    if (KS > 1 || WILDCAT_MFMA32_SCHEDBAR) __builtin_amdgcn_sched_barrier(0);
    if (Cfg::NBUF == 1) {
      // Private single buffer: the wave's own reads of this tile were issued
      // before these stores, and one wave's LDS accesses execute in order.
      store_tile(0);
    } else if (prefetch) {
      store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // eacc: partial over this lane's half of the keys -> full sum for row r32.
  eacc += __shfl_xor(eacc, 32, 64);
  if (KS > 1) {
    // Partial sums of the KS key ranges, [wave][value][lane], then added in
    // the order ks = 0, 1, ..., KS-1 by the waves of range 0.
    constexpr int NV = 16 * CT + 1;
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((size_t)wave * NV + 16 * ct + v) * 64 + lane] = oacc[ct][v];
    red[((size_t)wave * NV + 16 * CT) * 64 + lane] = eacc;
    __syncthreads();
    if (ks != 0) return;
#pragma unroll 1
    for (int q = 1; q < KS; ++q) {
      const size_t w2 = (size_t)q * Cfg::RW + rw;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[ct][v] += red[(w2 * NV + 16 * ct + v) * 64 + lane];
      eacc += red[(w2 * NV + 16 * CT) * 64 + lane];
    }
  }
  // oacc[ct][v] = result for left row 8 (v/4) + 4 g2 + v % 4 (of the wave's 32),
  // column 32 ct + r32.
  if (MODE == kModeWeights) {
    float* Y = p.out + ((size_t)split * p.units + unit) * p.rowsA * (D + 1);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = a0 + rw * 32 + 8 * (v >> 2) + 4 * g2 + (v & 3);
      if (row < p.rowsA) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Y[(size_t)row * (D + 1) + 32 * ct + r32] = oacc[ct][v];
      }
    }
    if (g2 == 0 && arow < p.rowsA) Y[(size_t)arow * (D + 1) + D] = eacc;
  } else {
    float* O = p.out + (size_t)unit * p.rowsA * D;
    // The lane's column bounds, read once (O stores could alias them, so
    // reading inside the store loop would reload them after every store);
    // per left row with range_rows.
    float lo[CT], hi[CT];
    if (!p.range_rows) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        lo[ct] = p.vmin[(size_t)unitB * D + 32 * ct + r32];
        hi[ct] = p.vmax[(size_t)unitB * D + 32 * ct + r32];
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = 8 * (v >> 2) + 4 * g2 + (v & 3);
      const float e = __shfl(eacc, rl, 64);
      const int row = a0 + rw * 32 + rl;
      if (row < p.rowsA) {
        if (p.range_rows) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const size_t k = ((size_t)unitB * p.rowsA + row) * D + 32 * ct + r32;
            lo[ct] = p.vmin[k];
            hi[ct] = p.vmax[k];
          }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          O[(size_t)row * D + 32 * ct + r32] = fminf(fmaxf(oacc[ct][v] / e, lo[ct]), hi[ct]);
      }
    }
  }
}

// fp32 inputs: the same contraction on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32, fp32 products and sums; P stays fp32).  A
// workgroup of NW waves owns 16 left rows per wave (their fragments in
// registers) and streams the right operand through LDS in tiles of KT rows.
// Per 16 right rows a wave issues
//   scores^T (16 right x 16 left) : D/4 MFMAs over d  -> lane (r16, g) holds
//                                   the scores of left row r16 with right
//                                   rows 4g .. 4g + 3
//   P = exp2(...) in fp32, masked
//   P x [V] (16 left x 16 cols)   : 4 MFMAs per 16 columns, MFMA v taking
//                                   right rows {4g + v}: P never leaves the
//                                   registers
// and the last column ([.., 1] or w) on the vector ALU.  LDS rows have a
// pitch of D + 4 floats, which keeps both the score and the value reads
// free of bank conflicts.  Output rows of the 16x16x4 MFMA: element v of
// lane (r16, g) is row 4g + v, column r16.
template <int D, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void expmm_f32m(ContractArgs p) {
  constexpr int NTH = 64 * NW;
  constexpr int KT = 64;             // right rows per LDS tile
  constexpr int KP = D + 4;          // LDS pitch (floats)
  constexpr int DC = D / 4;          // score MFMAs per 16 right rows
  constexpr int CT = D / 16;         // value column tiles
  __shared__ __attribute__((aligned(16))) float sB[KT * KP];
  __shared__ __attribute__((aligned(16))) float sV[KT * KP];
  __shared__ float sE[KT];           // attend: w; weights: 1 on valid rows
  __shared__ float sC[KT];           // weights: per-key offsets * log2(e)

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int unit = blockIdx.z, unitB = unit / p.group;
  const int a0 = blockIdx.y * 16 * NW;
  const int split = blockIdx.x;
  const int b_begin = MODE == kModeWeights ? split * p.chunk : 0;
  int b_end = MODE == kModeWeights ? min(p.rowsB, b_begin + p.chunk) : p.rowsB;
  if (MODE == kModeAttend && p.causal) b_end = min(b_end, p.causal_from + a0 + 16 * NW);

  const float* A = reinterpret_cast<const float*>(p.A) + (size_t)unit * p.rowsA * D;
  const float* B = reinterpret_cast<const float*>(p.B) + (size_t)unitB * p.rowsB * D;
  // left-row fragments (B operand of the score MFMA): row a0 + 16 wave + r16, d = 4 dc + g
  const int arow = a0 + wave * 16 + r16;
  float afrag[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) afrag[dc] = arow < p.rowsA ? A[(size_t)arow * D + 4 * dc + g] : 0.0f;
  float rc2 = 0.0f;
  if (MODE == kModeWeights && p.rowc != nullptr && arow < p.rowsA) rc2 = p.rowc[(size_t)unit * p.rowsA + arow] * kLog2e;
  const float sc2 = p.scale * kLog2e;

  f32x4 oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float eacc = 0.0f;

  for (int b0 = b_begin; b0 < b_end; b0 += KT) {
    // ---- stage the right tile and its values (zeros past b_end)
    for (int q = t; q < KT * (D / 4); q += NTH) {
      const int row = q / (D / 4), c4 = q % (D / 4);
      const int b = b0 + row;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (b < b_end) {
        kv = *reinterpret_cast<const float4*>(B + (size_t)b * D + 4 * c4);
        if (MODE == kModeWeights) {
          vv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.Vs) +
                                                ((size_t)unitB * p.rowsB + b) * D + 4 * c4);
        } else {
          const float* X = reinterpret_cast<const float*>(p.Vs) + ((size_t)unitB * p.rowsB + b) * (D + 1) + 4 * c4;
          vv = make_float4(X[0], X[1], X[2], X[3]);
        }
      }
      *reinterpret_cast<float4*>(&sB[row * KP + 4 * c4]) = kv;
      *reinterpret_cast<float4*>(&sV[row * KP + 4 * c4]) = vv;
    }
    for (int q = t; q < KT; q += NTH) {
      const int b = b0 + q;
      if (MODE == kModeAttend) {
        sE[q] = b < b_end ? reinterpret_cast<const float*>(p.Vs)[((size_t)unitB * p.rowsB + b) * (D + 1) + D] : 0.0f;
      } else {
        sE[q] = b < b_end ? 1.0f : 0.0f;
        sC[q] = (p.colc != nullptr && b < b_end) ? p.colc[(size_t)unitB * p.rowsB + b] * kLog2e : 0.0f;
      }
    }
    __syncthreads();

#pragma unroll
    for (int kb = 0; kb < KT / 16; ++kb) {
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(sB[(16 * kb + r16) * KP + 4 * dc + g], afrag[dc], s4, 0, 0, 0);
      // s4[v] = score of left row r16 with right row 16 kb + 4 g + v
      float pv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kk = 16 * kb + 4 * g + v;
        float arg = fmaf(s4[v], sc2, rc2);
        if (MODE == kModeWeights) arg += sC[kk];
        const bool keep = MODE == kModeWeights ? sE[kk] != 0.0f
                                               : (b0 + kk < b_end && visible(p, b0 + kk, arow));
        pv[v] = keep ? exp2f(arg) : 0.0f;
        eacc = fmaf(pv[v], sE[kk], eacc);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[v], sV[(16 * kb + 4 * g + v) * KP + 16 * ct + r16],
                                                          oacc[ct], 0, 0, 0);
    }
    __syncthreads();
  }

  // eacc: partial over this lane's right rows -> full sum for left row r16.
  eacc += __shfl_xor(eacc, 16, 64);
  eacc += __shfl_xor(eacc, 32, 64);

  // oacc[ct][v] = result for left row 16 wave + 4 g + v, column 16 ct + r16.
  if (MODE == kModeWeights) {
    float* Y = p.out + ((size_t)split * p.units + unit) * p.rowsA * (D + 1);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = a0 + wave * 16 + 4 * g + v;
      if (row < p.rowsA) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Y[(size_t)row * (D + 1) + 16 * ct + r16] = oacc[ct][v];
      }
    }
    if (g == 0 && arow < p.rowsA) Y[(size_t)arow * (D + 1) + D] = eacc;
  } else {
    float* O = p.out + (size_t)unit * p.rowsA * D;
    float lo[CT], hi[CT];   // read before any store: O stores could alias them
    if (!p.range_rows) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        lo[ct] = p.vmin[(size_t)unitB * D + 16 * ct + r16];
        hi[ct] = p.vmax[(size_t)unitB * D + 16 * ct + r16];
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rl = 4 * g + v;
      const float e = __shfl(eacc, rl, 64);
      const int row = a0 + wave * 16 + rl;
      if (row < p.rowsA) {
        if (p.range_rows) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const size_t k = ((size_t)unitB * p.rowsA + row) * D + 16 * ct + r16;
            lo[ct] = p.vmin[k];
            hi[ct] = p.vmax[k];
          }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          O[(size_t)row * D + 16 * ct + r16] = fminf(fmaxf(oacc[ct][v] / e, lo[ct]), hi[ct]);
      }
    }
  }
}

// K_S[u][j] = K[u][S[u][j]] for j < r_eff, zero rows after; optional per-pivot
// exponent offsets for recentring: rowc = c (|kbar|^2 - <k_s, kbar>).  Also
// initialises the value-range slots that value_range_part reduces into.
template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void gather_pivots(const TK* K, const int32_t* S, const int32_t* r_eff,
                                                        TK* K_S, const double* kbar, float* rowc,
                                                        int n, int r, double c, int* mmslot) {
  __shared__ double red[kBlock];
  const int u = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  // the value-range slots of unit u start at the identities of min / max
  if (j == 0)
    for (int e = t; e < 2 * D; e += kBlock) mmslot[(size_t)u * 2 * D + e] = e < D ? 0x7FFFFFFF : (int)0x80000000;
  const bool live = j < r_eff[u];
  const int s = live ? S[(size_t)u * r + j] : 0;
  for (int e = t; e < D; e += kBlock) {
    TK x;
    if (live) x = K[((size_t)u * n + s) * D + e];
    else memset(&x, 0, sizeof(TK));
    K_S[((size_t)u * r + j) * D + e] = x;
  }
  if (rowc != nullptr) {
    double acc = 0.0;
    for (int e = t; e < D; e += kBlock) {
      const double kb = kbar[(size_t)u * D + e];
      const double x = live ? (double)Elem<TK>::f32(K, ((size_t)u * n + s) * D + e) : 0.0;
      acc += kb * kb - x * kb;
    }
    red[t] = acc;
    __syncthreads();
    if (t == 0) {
      double sum = 0.0;
      for (int q = 0; q < kBlock; ++q) sum += red[q];
      rowc[(size_t)u * r + j] = live ? (float)(c * sum) : 0.0f;
    }
  }
}

// Per-key exponent offsets for recentring: colc = -c <kbar, k_l>.  Thread l
// reads its key row with 16-byte loads, all issued before the fp64 dot
// product (kbar staged in LDS).
template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void key_offsets(const TK* K, const double* kbar, float* colc, int n, double c) {
  constexpr int G = 16 / sizeof(TK), NG = D / G;
  __shared__ double sk[D];
  const int u = blockIdx.y;
  for (int e = threadIdx.x; e < D; e += kBlock) sk[e] = kbar[(size_t)u * D + e];
  __syncthreads();
  const int l = blockIdx.x * kBlock + threadIdx.x;
  const TK* row = K + ((size_t)u * n + min(l, n - 1)) * D;
  uint4 raw[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) raw[g] = *reinterpret_cast<const uint4*>(row + g * G);
  double acc = 0.0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t w[4] = {raw[g].x, raw[g].y, raw[g].z, raw[g].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (G == 8) {
        acc = fma((double)__uint_as_float(w[q] << 16), sk[g * G + 2 * q], acc);
        acc = fma((double)__uint_as_float(w[q] & 0xFFFF0000u), sk[g * G + 2 * q + 1], acc);
      } else {
        acc = fma((double)__uint_as_float(w[q]), sk[g * G + q], acc);
      }
    }
  }
  if (l < n) colc[(size_t)u * n + l] = (float)(-c * acc);
}

// Column min / max of V.  Workgroup (blk, u) covers rows [blk R, blk R + R),
// R = kMinMaxRows: thread t reads the 16-byte group t % NG of rows t / NG + RP p
// (RP = 256 / NG rows per pass), UNR loads issued before their min / max;
// rows past n re-read row n-1 (harmless for a min / max).  The RP row phases
// meet in LDS, then one integer atomic min / max per column on the
// order-encoded value (slots initialised by gather_pivots, decoded by the
// solve's first launch).
#ifndef WILDCAT_VR_UNR
#define WILDCAT_VR_UNR 8   // loads in flight per thread
#endif
template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void value_range_part(const TK* V, int* slot, int n) {
  constexpr int G = 16 / sizeof(TK);   // elements per 16 bytes
  constexpr int NG = D / G;            // groups per row
  constexpr int RP = kBlock / NG;      // rows per pass
  constexpr int NPASS = kMinMaxRows / RP;
  constexpr int UNR = NPASS < WILDCAT_VR_UNR ? NPASS : WILDCAT_VR_UNR;
  static_assert(NPASS % UNR == 0, "passes");
  __shared__ float smn[RP][D + 1], smx[RP][D + 1];
  const int u = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
  const int grp = t % NG, ph = t / NG;
  const int l0 = blk * kMinMaxRows;
  const TK* Vu = V + (size_t)u * n * D + grp * G;
  float mn[G], mx[G];
#pragma unroll
  for (int q = 0; q < G; ++q) { mn[q] = INFINITY; mx[q] = -INFINITY; }
#pragma unroll 1
  for (int p0 = 0; p0 < NPASS; p0 += UNR) {
    uint4 raw[UNR];
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int l = min(l0 + ph + RP * (p0 + j), n - 1);
      raw[j] = *reinterpret_cast<const uint4*>(Vu + (size_t)l * D);
    }
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      float x[G];
      if constexpr (G == 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[2 * q] = __uint_as_float(w[q] << 16);
          x[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = __uint_as_float(w[q]);
      }
#pragma unroll
      for (int q = 0; q < G; ++q) { mn[q] = fminf(mn[q], x[q]); mx[q] = fmaxf(mx[q], x[q]); }
    }
  }
#pragma unroll
  for (int q = 0; q < G; ++q) { smn[ph][grp * G + q] = mn[q]; smx[ph][grp * G + q] = mx[q]; }
  __syncthreads();
  for (int c = t; c < D; c += kBlock) {
    float a = INFINITY, b = -INFINITY;
    for (int p = 0; p < RP; ++p) { a = fminf(a, smn[p][c]); b = fmaxf(b, smx[p][c]); }
    atomicMin(&slot[((size_t)u * 2) * D + c], ord_enc(a));
    atomicMax(&slot[((size_t)u * 2 + 1) * D + c], ord_enc(b));
  }
}

// Binned RPNys: the value range of a unit is the min / max over its bins'
// ranges (bins in order; min and max are exact, so the order is immaterial).
__global__ __launch_bounds__(kBlock) void merge_ranges(const float* vmin_b, const float* vmax_b, float* vmin,
                                                       float* vmax, int units, int bins, int d) {
  const int e = blockIdx.x * kBlock + threadIdx.x;
  if (e >= units * d) return;
  const int u = e / d, c = e % d;
  float mn = vmin_b[((size_t)u * bins) * d + c], mx = vmax_b[((size_t)u * bins) * d + c];
  for (int b = 1; b < bins; ++b) {
    mn = fminf(mn, vmin_b[((size_t)u * bins + b) * d + c]);
    mx = fmaxf(mx, vmax_b[((size_t)u * bins + b) * d + c]);
  }
  vmin[e] = mn;
  vmax[e] = mx;
}

hipError_t launch_merge_ranges(int units, int bins, int d, const float* vmin_b, const float* vmax_b, float* vmin,
                               float* vmax, hipStream_t st) {
  merge_ranges<<<(unsigned)((units * d + kBlock - 1) / kBlock), kBlock, 0, st>>>(vmin_b, vmax_b, vmin, vmax, units,
                                                                                   bins, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------- host side
// Key split of the bf16 attend contraction (d >= 32): when the query row
// tiles alone give fewer than 256 workgroups (few query rows per head), a
// workgroup takes 32 query rows and its waves split the pivots into 8 ranges
// (d <= 64) or 4 ranges (d = 128), one wave per range.  Returns the number
// of ranges, 1 for no split.
inline int attend_key_split(int Uq, int m, int r, int d, bool bf16) {
  if (!bf16 || d < 32) return 1;
  const int rows = contract_rows_per_wg(d, m, true);
  const long wgs = (long)Uq * ((m + rows - 1) / rows);
  return (wgs < 256 && r >= 8 * 32) ? (d >= 128 ? 4 : 8) : 1;
}

// Grid: x = splits of the right rows, y = tiles of left rows, z = units.
// bf16 with d >= 32 runs the 32x32x16 kernel with 2, 4 or 8 waves (32 left
// rows each, see mfma32_waves), or for attend with few query rows the
// 8-wave key-split form (attend_key_split); bf16 d = 16 the 16x16x32 kernel;
// fp32 the 16x16x4 fp32 kernel.  contract_rows_per_wg gives the same tiling to
// the workspace layout.
template <int D, int MODE>
static void launch_expmm(bool bf16, const ContractArgs& a, int nsplit, hipStream_t st) {
  if constexpr (D >= 32 && MODE == kModeAttend) {
    const int ks = bf16 ? attend_key_split(a.units, a.rowsA, a.rowsB, D, true) : 1;
    if (ks > 1) {
      // One wave per key range, 32 query rows per workgroup.  d = 128 uses 4
      // waves: its staging registers need more than the 256 per lane that an
      // 8-wave workgroup allows.
      constexpr int KS = D >= 128 ? 4 : 8;
      expmm32<D, MODE, KS, false, KS><<<dim3(1, (a.rowsA + 31) / 32, a.units), 64 * KS, 0, st>>>(a);
      return;
    }
  }
  const int rows = contract_rows_per_wg(D, a.rowsA, bf16);
  const dim3 grid(nsplit, (a.rowsA + rows - 1) / rows, a.units);
  if (bf16) {
    if constexpr (D >= 32) {
      const int nw = mfma32_waves(a.rowsA);
      if (MODE == kModeWeights && a.colc != nullptr) {   // recentring offsets (weights only)
        constexpr bool RC = MODE == kModeWeights;
        if (nw == 8) expmm32<D, MODE, 8, RC, 1><<<grid, 512, 0, st>>>(a);
        else if (nw == 4) expmm32<D, MODE, 4, RC, 1><<<grid, 256, 0, st>>>(a);
        else expmm32<D, MODE, 2, RC, 1><<<grid, 128, 0, st>>>(a);
      } else {
        if (nw == 8) expmm32<D, MODE, 8, false, 1><<<grid, 512, 0, st>>>(a);
        else if (nw == 4) expmm32<D, MODE, 4, false, 1><<<grid, 256, 0, st>>>(a);
        else expmm32<D, MODE, 2, false, 1><<<grid, 128, 0, st>>>(a);
      }
    } else {
      expmm_bf16<D, MODE, 4><<<grid, 256, 0, st>>>(a);
    }
  } else {
    expmm_f32m<D, MODE, 4><<<grid, 256, 0, st>>>(a);
  }
}

template <int MODE>
static hipError_t launch_expmm_d(bool bf16, int d, const ContractArgs& a, int nsplit, hipStream_t st) {
  switch (d) {
    case 16: launch_expmm<16, MODE>(bf16, a, nsplit, st); break;
    case 32: launch_expmm<32, MODE>(bf16, a, nsplit, st); break;
    case 64: launch_expmm<64, MODE>(bf16, a, nsplit, st); break;
    case 128: launch_expmm<128, MODE>(bf16, a, nsplit, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TK, int D>
static void launch_weights_prep(int U, int n, int r, double c, int recentre, const void* K, const void* V,
                                const int32_t* S, const int32_t* r_eff, void* K_S, const WeightsLayout& lay,
                                char* w, float* vmin, float* vmax, hipStream_t st) {
  const TK* Kt = reinterpret_cast<const TK*>(K);
  double* kbar = reinterpret_cast<double*>(w + lay.kbar);
  float* rowc = reinterpret_cast<float*>(w + lay.rowc);
  float* colc = reinterpret_cast<float*>(w + lay.colc);
  if (recentre) {
    launch_key_mean<TK, D>(Kt, reinterpret_cast<double*>(w + lay.kpart), kbar, U, n, st);
    key_offsets<TK, D><<<dim3((n + kBlock - 1) / kBlock, U), kBlock, 0, st>>>(Kt, kbar, colc, n, c);
  }
  int* mm = reinterpret_cast<int*>(w + lay.mmslot);
  gather_pivots<TK, D><<<dim3(r, U), kBlock, 0, st>>>(Kt, S, r_eff, reinterpret_cast<TK*>(K_S), kbar,
                                                       recentre ? rowc : nullptr, n, r, c, mm);
  value_range_part<TK, D><<<dim3(lay.nmm, U), kBlock, 0, st>>>(reinterpret_cast<const TK*>(V), mm, n);
}

template <typename TK>
static hipError_t launch_prep_d(int d, int U, int n, int r, double c, int recentre, const void* K, const void* V,
                                const int32_t* S, const int32_t* r_eff, void* K_S, const WeightsLayout& lay,
                                char* w, float* vmin, float* vmax, hipStream_t st) {
  switch (d) {
    case 16: launch_weights_prep<TK, 16>(U, n, r, c, recentre, K, V, S, r_eff, K_S, lay, w, vmin, vmax, st); break;
    case 32: launch_weights_prep<TK, 32>(U, n, r, c, recentre, K, V, S, r_eff, K_S, lay, w, vmin, vmax, st); break;
    case 64: launch_weights_prep<TK, 64>(U, n, r, c, recentre, K, V, S, r_eff, K_S, lay, w, vmin, vmax, st); break;
    case 128: launch_weights_prep<TK, 128>(U, n, r, c, recentre, K, V, S, r_eff, K_S, lay, w, vmin, vmax, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_trsm(int U, int r, int d, const float* ypart, int nsplit, const double* L, const int32_t* r_eff,
                       float* X, float* vmin, float* vmax, const WeightsLayout& lay, char* ws, hipStream_t st);

// CompressKV after selection: K_S, value range, Y = h_tau(K_S, K) [V, 1], X.
hipError_t launch_weights(int bf16, int U, int n, int d, int r, double c, int recentre, const void* K,
                          const void* V, const int32_t* S, const int32_t* r_eff, const double* L, void* K_S,
                          float* X, float* vmin, float* vmax, void* ws, hipStream_t st) {
  const WeightsLayout lay(U, n, d, r, bf16 != 0);
  char* w = static_cast<char*>(ws);
  hipError_t e = bf16 ? launch_prep_d<bf16_t>(d, U, n, r, c, recentre, K, V, S, r_eff, K_S, lay, w, vmin, vmax, st)
                      : launch_prep_d<float>(d, U, n, r, c, recentre, K, V, S, r_eff, K_S, lay, w, vmin, vmax, st);
  if (e != hipSuccess) return e;
  ContractArgs a{};
  a.A = K_S; a.B = K; a.Vs = V;
  a.rowc = recentre ? reinterpret_cast<const float*>(w + lay.rowc) : nullptr;
  a.colc = recentre ? reinterpret_cast<const float*>(w + lay.colc) : nullptr;
  a.out = reinterpret_cast<float*>(w + lay.ypart);
  a.rowsA = r; a.rowsB = n; a.chunk = lay.sp.chunk; a.group = 1; a.units = U;
  a.scale = (float)c;
  e = launch_expmm_d<kModeWeights>(bf16 != 0, d, a, lay.sp.nsplit, st);
  if (e != hipSuccess) return e;
  return launch_trsm(U, r, d, a.out, lay.sp.nsplit, L, r_eff, X, vmin, vmax, lay, w, st);
}

// WtdAttn: O = clip(h(Q, K_S) X / (h(Q, K_S) w)).
hipError_t launch_attend(int bf16, int Uq, int group, int m, int d, int r, double beta, const void* Q,
                         const void* K_S, const float* X, const float* vmin, const float* vmax, float* O,
                         hipStream_t st) {
  ContractArgs a{};
  a.A = Q; a.B = K_S; a.Vs = X; a.out = O; a.vmin = vmin; a.vmax = vmax;
  a.rowsA = m; a.rowsB = r; a.chunk = r; a.group = group; a.units = Uq;
  a.scale = (float)beta;
  return launch_expmm_d<kModeAttend>(bf16 != 0, d, a, 1, st);
}

// ---- generation over a compressed cache --------------------------------
// [WildCat, KV-cache paragraph: the compressed keys and values enter the
// decoding phase through WtdAttn; m new tokens cost O(rmd + m^2 d).]
// New token j joins the weighted attention as a weight-1 point with value
// v_j, seen by the queries of tokens i >= j; the clip range of query i is
// the cache's range widened by v_0 .. v_i.  The cache and the new tokens are
// staged into one right operand ([K_S; K_new], [X; [V_new, 1]]) and attend
// runs over it with the causal mask from row r and a clip range per row.

// The running clip range over blocks of kRangeRows new values (fmin / fmax
// throughout: NaN values are skipped):
//   range_blocks: bmin[u][b][c], bmax = column extremes of block b (b < nblk - 1);
//   range_prefix: in place, bmin[u][b][c] = fmin(vmin[u][c], blocks 0 .. b);
//   decode_prep (range role): lo[u][i][c] = fmin(vmin[u][c], v_0c .. v_ic), hi
//                 likewise, from the prefix of the blocks before row i's block.
// With m <= kRangeRows (one block) only decode_prep runs.
template <typename TK, int D>
__global__ __launch_bounds__(D) void range_blocks(const TK* Vn, float* bmin, float* bmax, int m, int nblk) {
  const int blk = blockIdx.x, u = blockIdx.y, c = threadIdx.x;
  const int i0 = blk * kRangeRows, i1 = min(m, i0 + kRangeRows);
  float lo = INFINITY, hi = -INFINITY;
  for (int i = i0; i < i1; ++i) {
    const float v = Elem<TK>::f32(Vn, ((size_t)u * m + i) * D + c);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  bmin[((size_t)u * nblk + blk) * D + c] = lo;
  bmax[((size_t)u * nblk + blk) * D + c] = hi;
}

template <int D>
__global__ __launch_bounds__(D) void range_prefix(const float* vmin, const float* vmax, float* bmin, float* bmax,
                                                  int nblk) {
  const int u = blockIdx.x, c = threadIdx.x;
  float lo = vmin[(size_t)u * D + c], hi = vmax[(size_t)u * D + c];
  for (int b = 0; b + 1 < nblk; ++b) {
    const size_t k = ((size_t)u * nblk + b) * D + c;
    lo = fminf(lo, bmin[k]);
    hi = fmaxf(hi, bmax[k]);
    bmin[k] = lo;
    bmax[k] = hi;
  }
}

constexpr int kPrepItems = 8;   // staged items per thread of decode_prep

struct DecodePrepArgs {
  const void *K_S, *Kn, *Vn;
  const float *X, *vmin, *vmax, *bmin, *bmax;
  void* keys;
  float *xs, *lo, *hi;
  int r, m, nblk, nstage;   // nstage: workgroups of the staging role
};

// One launch, two roles.  Workgroup b < nblk writes the running range of
// block b of the new tokens (thread c: column c; the block's values are
// loaded before the scan).  Workgroups nblk .. nblk + nstage - 1 stage the
// operand: keys[u] = [K_S[u]; K_new[u]], xs[u] = [X[u]; [V_new[u], 1]].
template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void decode_prep(DecodePrepArgs a) {
  const int u = blockIdx.y, t = threadIdx.x;
  const TK* Vn = reinterpret_cast<const TK*>(a.Vn);
  if ((int)blockIdx.x >= a.nblk) {
    // kPrepItems consecutive-by-thread items per thread; both candidate
    // sources are loaded at clamped (valid) indices and the right one is
    // selected, so no load waits behind a branch.
    const TK* K_S = reinterpret_cast<const TK*>(a.K_S);
    const TK* Kn = reinterpret_cast<const TK*>(a.Kn);
    TK* keys = reinterpret_cast<TK*>(a.keys);
    const int r = a.r, m = a.m;
    const int64_t R = (int64_t)r + m;
    const int64_t base = (int64_t)(blockIdx.x - a.nblk) * kBlock * kPrepItems + t;
    const float* Xu = a.X + (size_t)u * r * (D + 1);
    const TK* Vu = Vn + (size_t)u * m * D;
    const int64_t nx = R * (D + 1), nk = R * D, xlast = (int64_t)r * (D + 1) - 1, vlast = (int64_t)m * D - 1;
    float xv[kPrepItems];
#pragma unroll
    for (int k = 0; k < kPrepItems; ++k) {
      const int64_t idx = base + (int64_t)k * kBlock;
      const int64_t row = idx / (D + 1);
      const int c = (int)(idx - row * (D + 1));
      const float fx = Xu[std::min(std::max(idx, (int64_t)0), std::max(xlast, (int64_t)0))];
      const float fv = Elem<TK>::f32(Vu, std::min(std::max((row - r) * D + c, (int64_t)0), vlast));
      xv[k] = row < r ? fx : (c < D ? fv : 1.0f);
    }
#pragma unroll
    for (int k = 0; k < kPrepItems; ++k) {
      const int64_t idx = base + (int64_t)k * kBlock;
      if (idx < nx) a.xs[(size_t)u * R * (D + 1) + idx] = xv[k];
    }
    const TK* Ku = K_S + (size_t)u * r * D;
    const TK* Knu = Kn + (size_t)u * m * D;
    const int64_t klast = (int64_t)r * D - 1;
    TK kv[kPrepItems];
#pragma unroll
    for (int k = 0; k < kPrepItems; ++k) {
      const int64_t idx = base + (int64_t)k * kBlock;
      const TK ks = Ku[std::min(std::max(idx, (int64_t)0), std::max(klast, (int64_t)0))];
      const TK kn = Knu[std::min(std::max(idx - (int64_t)r * D, (int64_t)0), vlast)];
      kv[k] = idx < (int64_t)r * D ? ks : kn;
    }
#pragma unroll
    for (int k = 0; k < kPrepItems; ++k) {
      const int64_t idx = base + (int64_t)k * kBlock;
      if (idx < nk) keys[(size_t)u * R * D + idx] = kv[k];
    }
    return;
  }
  const int blk = blockIdx.x, c = t;
  if (c >= D) return;
  float lo, hi;
  if (blk == 0) {
    lo = a.vmin[(size_t)u * D + c];
    hi = a.vmax[(size_t)u * D + c];
  } else {
    lo = a.bmin[((size_t)u * a.nblk + blk - 1) * D + c];
    hi = a.bmax[((size_t)u * a.nblk + blk - 1) * D + c];
  }
  const int i0 = blk * kRangeRows, cnt = min(a.m - i0, kRangeRows);
  // unconditional loads (rows past the end re-read the last row): a branch
  // around each load would make every one wait for the previous
  float v[kRangeRows];
#pragma unroll
  for (int j = 0; j < kRangeRows; ++j) v[j] = Elem<TK>::f32(Vn, ((size_t)u * a.m + i0 + min(j, cnt - 1)) * D + c);
#pragma unroll
  for (int j = 0; j < kRangeRows; ++j) {
    if (j < cnt) {
      const size_t k = ((size_t)u * a.m + i0 + j) * D + c;
      lo = fminf(lo, v[j]);
      hi = fmaxf(hi, v[j]);
      a.lo[k] = lo;
      a.hi[k] = hi;
    }
  }
}

template <typename TK, int D>
static void launch_decode_prep(int Ukv, int m, int r, const void* K_S, const float* X, const void* Kn, const void* Vn,
                               const float* vmin, const float* vmax, const DecodeLayout& lay, char* w,
                               hipStream_t st) {
  DecodePrepArgs a{};
  a.K_S = K_S; a.Kn = Kn; a.Vn = Vn; a.X = X; a.vmin = vmin; a.vmax = vmax;
  float* bmin = reinterpret_cast<float*>(w + lay.bmin);
  float* bmax = reinterpret_cast<float*>(w + lay.bmax);
  a.bmin = bmin; a.bmax = bmax;
  a.keys = w + lay.keys;
  a.xs = reinterpret_cast<float*>(w + lay.xs);
  a.lo = reinterpret_cast<float*>(w + lay.lo);
  a.hi = reinterpret_cast<float*>(w + lay.hi);
  a.r = r; a.m = m; a.nblk = lay.nblk;
  const int64_t items = ((int64_t)r + m) * (D + 1);
  a.nstage = (int)((items + kBlock * kPrepItems - 1) / (kBlock * kPrepItems));
  if (lay.nblk > 1) {
    const TK* V = reinterpret_cast<const TK*>(Vn);
    range_blocks<TK, D><<<dim3(lay.nblk - 1, Ukv), D, 0, st>>>(V, bmin, bmax, m, lay.nblk);
    range_prefix<D><<<Ukv, D, 0, st>>>(vmin, vmax, bmin, bmax, lay.nblk);
  }
  decode_prep<TK, D><<<dim3(lay.nblk + a.nstage, Ukv), kBlock, 0, st>>>(a);
}

// One new token (m = 1), the usual step of token-by-token generation: no
// staging of the cache (the general form copies it into its operand and runs
// a 32-row tile for one query row).  decode_one_part: workgroup (s, q-head)
// takes key range s of the cache (one_token_split ranges of about 128 keys,
// so the cache of a head is read by several CUs at once).  Phase 1: the
// kernel values of its keys in fp32 (fp32 dot products of the exact inputs,
// exp2), kept in LDS; range 0 also computes the new token's.  Phase 2: the
// 256 threads split into D/4 column quads x 1024/D sub-ranges (16-byte loads
// of X rows, which are 4-byte aligned; the weight column by the quad-0
// threads); the sub-ranges' sums are added in order and written out.
// decode_one_final: N = the ranges' sums in order + p_new [v_new, 1], then
// O = clip(N[:d] / N[d]) with the range widened by v_new.
template <typename TK, int D>
__device__ __forceinline__ float dot_row(const TK* k, const float* sq) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if constexpr (std::is_same<TK, bf16_t>::value) {
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(k + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = __uint_as_float(w[j] << 16), x1 = __uint_as_float(w[j] & 0xFFFF0000u);
        if (j & 1) { a2 = fmaf(x0, sq[c + 2 * j], a2); a3 = fmaf(x1, sq[c + 2 * j + 1], a3); }
        else { a0 = fmaf(x0, sq[c + 2 * j], a0); a1 = fmaf(x1, sq[c + 2 * j + 1], a1); }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const float4 v = *reinterpret_cast<const float4*>(k + c);
      a0 = fmaf(v.x, sq[c], a0); a1 = fmaf(v.y, sq[c + 1], a1);
      a2 = fmaf(v.z, sq[c + 2], a2); a3 = fmaf(v.w, sq[c + 3], a3);
    }
  }
  return (a0 + a1) + (a2 + a3);
}

template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void decode_one_part(const TK* Q, const TK* K_S, const float* X, const TK* Kn,
                                                          float* part, float* pnew, int r, int group, int S,
                                                          float scale2) {
  constexpr int NQ = D / 4, NR = kBlock / NQ;   // column quads, sub-ranges
  extern __shared__ float dsm[];
  const int s = blockIdx.x, uq = blockIdx.y, u = uq / group, t = threadIdx.x;
  const int k0 = (int)((int64_t)r * s / S), k1 = (int)((int64_t)r * (s + 1) / S), nk = k1 - k0;
  float* sp = dsm;                              // nk kernel values
  float* sq = dsm + ((nk + 3) & ~3);            // D query values
  float* red = sq + D;                          // [NR][D + 1] sub-range sums
  for (int c = t; c < D; c += kBlock) sq[c] = Elem<TK>::f32(Q, (size_t)uq * D + c);
  __syncthreads();
  for (int l = t; l < nk; l += kBlock) sp[l] = exp2f(dot_row<TK, D>(K_S + ((size_t)u * r + k0 + l) * D, sq) * scale2);
  if (s == 0 && t == 0) pnew[uq] = exp2f(dot_row<TK, D>(Kn + (size_t)u * D, sq) * scale2);
  __syncthreads();
  const int cq = t % NQ, kr = t / NQ;
  const int l0 = k0 + (int)((int64_t)nk * kr / NR), l1 = k0 + (int)((int64_t)nk * (kr + 1) / NR);
  typedef float f4a __attribute__((ext_vector_type(4), aligned(4)));
  const float* Xu = X + (size_t)u * r * (D + 1);
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, accw = 0.f;
  int l = l0;
#pragma unroll 1
  for (; l + 8 <= l1; l += 8) {
    f4a x[8];
    float xw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      x[q] = *reinterpret_cast<const f4a*>(Xu + (size_t)(l + q) * (D + 1) + 4 * cq);
      xw[q] = Xu[(size_t)(l + q) * (D + 1) + D];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float p = sp[l + q - k0];
      acc[0] = fmaf(p, x[q].x, acc[0]); acc[1] = fmaf(p, x[q].y, acc[1]);
      acc[2] = fmaf(p, x[q].z, acc[2]); acc[3] = fmaf(p, x[q].w, acc[3]);
      accw = fmaf(p, xw[q], accw);
    }
  }
  for (; l < l1; ++l) {
    const f4a x = *reinterpret_cast<const f4a*>(Xu + (size_t)l * (D + 1) + 4 * cq);
    const float p = sp[l - k0];
    acc[0] = fmaf(p, x.x, acc[0]); acc[1] = fmaf(p, x.y, acc[1]);
    acc[2] = fmaf(p, x.z, acc[2]); acc[3] = fmaf(p, x.w, acc[3]);
    accw = fmaf(p, Xu[(size_t)l * (D + 1) + D], accw);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[kr * (D + 1) + 4 * cq + j] = acc[j];
  if (cq == 0) red[kr * (D + 1) + D] = accw;
  __syncthreads();
  for (int c = t; c <= D; c += kBlock) {
    float n = 0.f;
    for (int k = 0; k < NR; ++k) n += red[k * (D + 1) + c];
    part[((size_t)uq * kOneSplit + s) * (D + 1) + c] = n;
  }
}

template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void decode_one_final(const float* part, const float* pnew, const float* vmin,
                                                           const float* vmax, const TK* Vn, float* O, int group,
                                                           int S) {
  __shared__ float sN[D + 1];
  const int uq = blockIdx.x, u = uq / group, t = threadIdx.x;
  for (int c = t; c <= D; c += kBlock) {
    float n = 0.f;
    for (int s = 0; s < S; ++s) n += part[((size_t)uq * kOneSplit + s) * (D + 1) + c];
    const float vn = c < D ? Elem<TK>::f32(Vn, (size_t)u * D + c) : 1.0f;
    sN[c] = fmaf(pnew[uq], vn, n);
  }
  __syncthreads();
  for (int c = t; c < D; c += kBlock) {
    const float vn = Elem<TK>::f32(Vn, (size_t)u * D + c);
    const float lo = fminf(vmin[(size_t)u * D + c], vn), hi = fmaxf(vmax[(size_t)u * D + c], vn);
    O[(size_t)uq * D + c] = fminf(fmaxf(sN[c] / sN[D], lo), hi);
  }
}

template <typename TK, int D>
static void launch_decode_one(int Uq, int group, int r, double beta, const void* Q, const void* K_S, const float* X,
                              const float* vmin, const float* vmax, const void* Kn, const void* Vn, float* O,
                              const DecodeLayout& lay, char* w, hipStream_t st) {
  constexpr int NR = kBlock / (D / 4);
  const int S = one_token_split(r);
  const int nkmax = (r + S - 1) / S;
  const size_t lds = (((nkmax + 3) & ~3) + D + NR * (D + 1)) * sizeof(float);
  float* part = reinterpret_cast<float*>(w + lay.part);
  float* pnew = reinterpret_cast<float*>(w + lay.pnew);
  decode_one_part<TK, D><<<dim3(S, Uq), kBlock, lds, st>>>(
      reinterpret_cast<const TK*>(Q), reinterpret_cast<const TK*>(K_S), X, reinterpret_cast<const TK*>(Kn), part, pnew,
      r, group, S, (float)beta * kLog2e);
  decode_one_final<TK, D><<<Uq, kBlock, 0, st>>>(part, pnew, vmin, vmax, reinterpret_cast<const TK*>(Vn), O, group,
                                                 S);
}

// Decode: O = clip(N[:, :d] / N[:, d]) with N_i = h(q_i, K_S) X + sum_{j<=i} h(q_i, k_j) [v_j, 1].
hipError_t launch_decode(int bf16, int Uq, int group, int m, int d, int r, double beta, const void* Q,
                         const void* K_S, const float* X, const float* vmin, const float* vmax, const void* Kn,
                         const void* Vn, float* O, void* ws, hipStream_t st) {
  const int Ukv = Uq / group;
  const DecodeLayout lay(Ukv, m, d, r, bf16 != 0, Uq);
  char* w = static_cast<char*>(ws);
  if (m == 1) {
#define WC_DECODE_ONE(TK, DD) \
  launch_decode_one<TK, DD>(Uq, group, r, beta, Q, K_S, X, vmin, vmax, Kn, Vn, O, lay, w, st)
    switch (d) {
      case 16: if (bf16) WC_DECODE_ONE(bf16_t, 16); else WC_DECODE_ONE(float, 16); break;
      case 32: if (bf16) WC_DECODE_ONE(bf16_t, 32); else WC_DECODE_ONE(float, 32); break;
      case 64: if (bf16) WC_DECODE_ONE(bf16_t, 64); else WC_DECODE_ONE(float, 64); break;
      case 128: if (bf16) WC_DECODE_ONE(bf16_t, 128); else WC_DECODE_ONE(float, 128); break;
      default: return hipErrorInvalidValue;
    }
#undef WC_DECODE_ONE
    return hipGetLastError();
  }
#define WC_DECODE_PREP(TK, DD) launch_decode_prep<TK, DD>(Ukv, m, r, K_S, X, Kn, Vn, vmin, vmax, lay, w, st)
  switch (d) {
    case 16: if (bf16) WC_DECODE_PREP(bf16_t, 16); else WC_DECODE_PREP(float, 16); break;
    case 32: if (bf16) WC_DECODE_PREP(bf16_t, 32); else WC_DECODE_PREP(float, 32); break;
    case 64: if (bf16) WC_DECODE_PREP(bf16_t, 64); else WC_DECODE_PREP(float, 64); break;
    case 128: if (bf16) WC_DECODE_PREP(bf16_t, 128); else WC_DECODE_PREP(float, 128); break;
    default: return hipErrorInvalidValue;
  }
#undef WC_DECODE_PREP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ContractArgs a{};
  a.A = Q; a.B = w + lay.keys; a.Vs = w + lay.xs; a.out = O;
  a.vmin = reinterpret_cast<const float*>(w + lay.lo);
  a.vmax = reinterpret_cast<const float*>(w + lay.hi);
  a.rowsA = m; a.rowsB = r + m; a.chunk = r + m; a.group = group; a.units = Uq;
  a.scale = (float)beta;
  a.causal = 1; a.causal_from = r; a.range_rows = 1;
  return launch_expmm_d<kModeAttend>(bf16 != 0, d, a, 1, st);
}

}  // namespace wc
