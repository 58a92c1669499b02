// Launch geometry of the exp-kernel contractions and the weights workspace
// layout (host side).
#pragma once

#include "layout.hpp"

namespace wc {

// Geometry of the exp-kernel contractions.
constexpr int kTileRows = 64;   // left rows per workgroup of the 16x16 and fp32 kernels
constexpr int kTileKeys = 128;  // split chunks are multiples of this (the largest right-row tile)

// Waves per workgroup of the 32x32 bf16 kernel (32 left rows per wave).
#ifndef WILDCAT_MFMA32_MAXWAVES
#define WILDCAT_MFMA32_MAXWAVES 8
#endif
inline int mfma32_waves(int rowsA) {
  const int w = rowsA > 128 ? 8 : (rowsA > 64 ? 4 : 2);
  return w < WILDCAT_MFMA32_MAXWAVES ? w : WILDCAT_MFMA32_MAXWAVES;
}

// Left rows one workgroup owns, for the kernel that a (d, dtype, rows) call uses.
inline int contract_rows_per_wg(int d, int rowsA, bool bf16) {
  return (bf16 && d >= 32) ? 32 * mfma32_waves(rowsA) : kTileRows;
}

struct ContractSplit {
  int tiles_a, nsplit, chunk;   // chunk: keys per split, multiple of kTileKeys
  ContractSplit(int U, int r, int n, int rows_per_wg) {
    tiles_a = (r + rows_per_wg - 1) / rows_per_wg;
    // about one workgroup per CU (256 CUs) for the large-tile kernels
    int want = (256 + tiles_a * U - 1) / (tiles_a * U);
    int maxs = (n + kTileKeys - 1) / kTileKeys;
    nsplit = want < 1 ? 1 : (want > maxs ? maxs : want);
    chunk = ((n + nsplit - 1) / nsplit + kTileKeys - 1) / kTileKeys * kTileKeys;
    nsplit = (n + chunk - 1) / chunk;
  }
};

// Weights workspace:
//   ypart   [nsplit][U][r][d+1] fp32   split-n partial contractions
//   mmpart  [U][nmm][2][d]      fp32   partial column min / max of V
//   kbar    [U][d]              fp64   key mean (recentring only)
//   rowc    [U][r]              fp32   per-pivot exponent offsets (recentring only)
//   colc    [U][n]              fp32   per-key exponent offsets (recentring only)
//   LT      [U][r][r]           fp64   transposed pivot block for the forward solve
//   Dinv    [U][r/64+1][64][64] fp64   inverses of the 64x64 diagonal blocks of the pivot block
constexpr int kMinMaxRows = 1024;   // rows of V per min/max partial
struct WeightsLayout {
  ContractSplit sp;
  int nmm;
  size_t ypart, mmpart, kbar, rowc, colc, LT, Dinv, total;
  WeightsLayout(int U, int n, int d, int r, bool bf16) : sp(U, r, n, contract_rows_per_wg(d, r, bf16)) {
    nmm = (n + kMinMaxRows - 1) / kMinMaxRows;
    size_t o = 0;
    ypart = o;  o += al256((size_t)sp.nsplit * U * r * (d + 1) * 4);
    mmpart = o; o += al256((size_t)U * nmm * 2 * d * 4);
    kbar = o;   o += al256((size_t)U * d * 8);
    rowc = o;   o += al256((size_t)U * r * 4);
    colc = o;   o += al256((size_t)U * n * 4);
    LT = o;     o += al256((size_t)U * r * r * 8);
    Dinv = o;   o += al256((size_t)U * (r / 64 + 1) * 64 * 64 * 8);
    total = o;
  }
};

}  // namespace wc

namespace wc {

// Decode workspace (generation over a compressed cache with m new tokens).
// One new token (m = 1):
//   part    [Uq][kOneSplit][d+1] fp32  partial sums of each query head's key ranges
//   pnew    [Uq]                 fp32  kernel value of the new token
// m > 1:
//   keys    [U][r+m][d]       dtype  coreset keys, then the new tokens' keys
//   xs      [U][r+m][d+1]     fp32   X, then [v_j, 1] for the new tokens
//   lo, hi  [U][m][d]         fp32   running clip range of every new token
//   bmin, bmax [U][nblk][d]   fp32   minima / maxima of blocks of kRangeRows new values
constexpr int kRangeRows = 64;
constexpr int kOneSplit = 8;      // most key ranges per query head for one new token
constexpr int kOneKeys = 128;     // keys per range it aims at
inline int one_token_split(int r) {
  const int s = r / kOneKeys;
  return s < 1 ? 1 : (s > kOneSplit ? kOneSplit : s);
}
struct DecodeLayout {
  int nblk;
  size_t keys = 0, xs = 0, lo = 0, hi = 0, bmin = 0, bmax = 0, part = 0, pnew = 0, total;
  DecodeLayout(int U, int m, int d, int r, bool bf16, int Uq) {
    const size_t R = (size_t)r + m;
    nblk = (m + kRangeRows - 1) / kRangeRows;
    size_t o = 0;
    if (m == 1) {
      part = o; o += al256((size_t)Uq * kOneSplit * (d + 1) * 4);
      pnew = o; o += al256((size_t)Uq * 4);
      total = o;
      return;
    }
    keys = o; o += al256((size_t)U * R * d * (bf16 ? 2 : 4));
    xs = o;   o += al256((size_t)U * R * (d + 1) * 4);
    lo = o;   o += al256((size_t)U * m * d * 4);
    hi = o;   o += al256((size_t)U * m * d * 4);
    bmin = o; o += al256((size_t)U * nblk * d * 4);
    bmax = o; o += al256((size_t)U * nblk * d * 4);
    total = o;
  }
};

}  // namespace wc
