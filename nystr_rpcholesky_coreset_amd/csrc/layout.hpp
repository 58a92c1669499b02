// RPNys workspace layout and the size limits shared by the library (host side).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace wc {

constexpr int kSelRowsPerThread = 2;                        // fp64 rows per lane in the step kernel
constexpr int kSelRowsPerBlock = 64 * kSelRowsPerThread;    // rows of one workgroup (one wave's lanes) = one scan block
constexpr int kMaxR = 4096;
constexpr int kMaxN = 1 << 21;

inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// RPNys workspace for U units of n keys, rank r, head dim d, factor entries
// of fbytes bytes (8: float64, 4: float32 storage).
//   F      [U][nb][r][128] fp64 or fp32  factor, block-major: slab (u, blk) holds
//                                 columns 0..r-1 of the Cholesky factor for that block's 128 keys
//   dres   [U][npad]    fp64   residual diagonal (0 on padding rows)
//   bsum   [U][nb]      fp64   per-workgroup residual sums of the last step
//   pivbuf [U][2][pbs]  fp64   next pivot: s, sqrt(g_s), F[s,:i], k_s (double buffered by step parity)
//   T0     [U]          fp64   initial residual trace
//   kbar   [U][d]       fp64   key mean (recentring only)
//   kpart  [U][ceil(n/1024)][d] fp64  partial key sums (recentring only)
//   stopped, reff [U] int32
struct SelectLayout {
  int nb, npad, pbs;
  size_t F, dres, bsum, pivbuf, T0, kbar, kpart, stopped, reff, total;
  SelectLayout(int U, int n, int d, int r, int fbytes = 8) {
    nb = (n + kSelRowsPerBlock - 1) / kSelRowsPerBlock;
    npad = nb * kSelRowsPerBlock;
    pbs = (2 + r + d + 3) / 4 * 4;
    size_t o = 0;
    F = o;       o += al256((size_t)U * r * npad * fbytes);
    dres = o;    o += al256((size_t)U * npad * 8);
    bsum = o;    o += al256((size_t)U * nb * 8);
    pivbuf = o;  o += al256((size_t)U * 2 * pbs * 8);
    T0 = o;      o += al256((size_t)U * 8);
    kbar = o;    o += al256((size_t)U * d * 8);
    kpart = o;   o += al256((size_t)U * ((n + 1023) / 1024) * d * 8);
    stopped = o; o += al256((size_t)U * 4);
    reff = o;    o += al256((size_t)U * 4);
    total = o;
  }
};

}  // namespace wc
