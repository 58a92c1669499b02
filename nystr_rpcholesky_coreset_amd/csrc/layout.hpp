// Workspace layouts and launch geometry of the WildCat library (host side).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace wc {

constexpr int kSelRowsPerThread = 2;                        // fp64 rows per lane in the step kernel
constexpr int kSelRowsPerBlock = 64 * kSelRowsPerThread;    // rows of one workgroup (one wave's lanes) = one scan block
constexpr int kMaxR = 4096;
constexpr int kMaxN = 1 << 21;

inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// RPNys workspace for U units of n keys, rank r, head dim d.
//   F      [U][nb][r][128] fp64  factor, block-major: slab (u, blk) holds columns
//                                 0..r-1 of the Cholesky factor for that block's 128 keys
//   dres   [U][npad]    fp64   residual diagonal (0 on padding rows)
//   bsum   [U][nb]      fp64   per-workgroup residual sums of the last step
//   pivbuf [U][2][pbs]  fp64   next pivot: s, sqrt(g_s), F[s,:i], k_s (double buffered by step parity)
//   T0     [U]          fp64   initial residual trace
//   kbar   [U][d]       fp64   key mean (recentring only)
//   stopped, reff [U] int32
struct SelectLayout {
  int nb, npad, pbs;
  size_t F, dres, bsum, pivbuf, T0, kbar, stopped, reff, total;
  SelectLayout(int U, int n, int d, int r) {
    nb = (n + kSelRowsPerBlock - 1) / kSelRowsPerBlock;
    npad = nb * kSelRowsPerBlock;
    pbs = (2 + r + d + 3) / 4 * 4;
    size_t o = 0;
    F = o;       o += al256((size_t)U * r * npad * 8);
    dres = o;    o += al256((size_t)U * npad * 8);
    bsum = o;    o += al256((size_t)U * nb * 8);
    pivbuf = o;  o += al256((size_t)U * 2 * pbs * 8);
    T0 = o;      o += al256((size_t)U * 8);
    kbar = o;    o += al256((size_t)U * d * 8);
    stopped = o; o += al256((size_t)U * 4);
    reff = o;    o += al256((size_t)U * 4);
    total = o;
  }
};

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
//   Y       [U][r][d+1]         fp64   summed contraction h_tau(K_S, K) [V, 1]
constexpr int kMinMaxRows = 1024;   // rows of V per min/max partial
struct WeightsLayout {
  ContractSplit sp;
  int nmm;
  size_t ypart, mmpart, kbar, rowc, colc, LT, Y, total;
  WeightsLayout(int U, int n, int d, int r, bool bf16) : sp(U, r, n, contract_rows_per_wg(d, r, bf16)) {
    nmm = (n + kMinMaxRows - 1) / kMinMaxRows;
    size_t o = 0;
    ypart = o;  o += al256((size_t)sp.nsplit * U * r * (d + 1) * 4);
    mmpart = o; o += al256((size_t)U * nmm * 2 * d * 4);
    kbar = o;   o += al256((size_t)U * d * 8);
    rowc = o;   o += al256((size_t)U * r * 4);
    colc = o;   o += al256((size_t)U * n * 4);
    LT = o;     o += al256((size_t)U * r * r * 8);
    Y = o;      o += al256((size_t)U * r * (d + 1) * 8);
    total = o;
  }
};

}  // namespace wc
