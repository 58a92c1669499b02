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

// Geometry of the triangular solves: diagonal blocks of b rows (the rank
// padded to rp, a multiple of b), and the d+1 right-hand-side columns padded
// to cp = 16 nct, taken nc column tiles of 16 at a time.
#ifndef WILDCAT_SOLVE_BMAX
#define WILDCAT_SOLVE_BMAX 256   // largest diagonal block of the solves (a power of 2, 64 .. 256)
#endif
static_assert(WILDCAT_SOLVE_BMAX >= 64 && WILDCAT_SOLVE_BMAX <= 256, "diagonal blocks of 64 .. 256 rows");
struct SolveGeom {
  int b, rp, nct, cp, nc;
  SolveGeom(int r, int d) {
    b = 64;
    while (b < r && b < WILDCAT_SOLVE_BMAX) b *= 2;
    rp = (r + b - 1) / b * b;
    nct = (d + 1 + 15) / 16;      // 2, 3, 5, 9 for d = 16, 32, 64, 128
    cp = 16 * nct;
    nc = nct == 9 ? 3 : nct;
  }
};

// Weights workspace:
//   ypart   [nsplit][U][r][d+1] fp32   split-n partial contractions
//   mmslot  [U][2][d]           int32  column min / max of V, order-encoded (atomics)
//   kbar    [U][d]              fp64   key mean (recentring only)
//   kpart   [U][ceil(n/1024)][d] fp64  partial key sums (recentring only)
//   rowc    [U][r]              fp32   per-pivot exponent offsets (recentring only)
//   colc    [U][n]              fp32   per-key exponent offsets (recentring only)
//   band    [U][rp][b]          fp64   inverses of the b x b diagonal blocks of the pivot block
//   yw, zw  [U][rp][cp]         fp64   right-hand sides during the two sweeps (yw ends as X)
#ifndef WILDCAT_VR_ROWS
#define WILDCAT_VR_ROWS 512
#endif
constexpr int kMinMaxRows = WILDCAT_VR_ROWS;   // rows of V per value-range workgroup
struct WeightsLayout {
  ContractSplit sp;
  SolveGeom sg;
  int nmm;                          // value-range workgroups per unit
  size_t ypart, mmslot, kbar, kpart, rowc, colc, band, yw, zw, total;
  WeightsLayout(int U, int n, int d, int r, bool bf16)
      : sp(U, r, n, contract_rows_per_wg(d, r, bf16)), sg(r, d) {
    nmm = (n + kMinMaxRows - 1) / kMinMaxRows;
    size_t o = 0;
    ypart = o;  o += al256((size_t)sp.nsplit * U * r * (d + 1) * 4);
    mmslot = o; o += al256((size_t)U * 2 * d * 4);
    kbar = o;   o += al256((size_t)U * d * 8);
    kpart = o;  o += al256((size_t)U * ((n + 1023) / 1024) * d * 8);
    rowc = o;   o += al256((size_t)U * r * 4);
    colc = o;   o += al256((size_t)U * n * 4);
    band = o;   o += al256((size_t)U * sg.rp * sg.b * 8);
    yw = o;     o += al256((size_t)U * sg.rp * sg.cp * 8);
    zw = o;     o += al256((size_t)U * sg.rp * sg.cp * 8);
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
