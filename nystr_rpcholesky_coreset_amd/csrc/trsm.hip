// Nystroem weights through the pivot block: X = L^{-T} (L^{-1} Y), float64.
//
// [WildCat (arXiv 2602.10056), Nystroem and CompressKV / Alg. 2 paragraphs:
// W = h_tau(K_S, K_S)^{-1} h_tau(K_S, K); with h_tau(K_S, K_S) = L L^T from the
// Cholesky pivot block, W [V, 1] = L^{-T} L^{-1} (h_tau(K_S, K) [V, 1]).]
//
// Blocked by tiles of 64 rows with inverted diagonal blocks: one kernel
// inverts every 64x64 diagonal block of L (one wave per block, column j of
// the inverse by substitution in lane j, fp64); the solve then applies
// L_tt^{-1} (forward) and L_tt^{-T} (backward) to a tile as a small
// matrix-vector product, with no serial chain.  One workgroup of NT threads
// (256 for r <= 256, else 1024) per (unit, group of CPW right-hand-side
// columns), right-looking.  Thread t owns rows t, t + NT, ... of the
// right-hand sides and keeps them in registers for the whole solve, so the
// 64 rows of a tile belong to exactly one wave: that wave multiplies them by
// the staged inverse block and publishes the solved values to LDS; then
// every thread subtracts the tile's contribution from its own remaining rows,
// with independent coalesced loads (L^T rows in the forward sweep, L rows in
// the backward sweep: consecutive threads read consecutive doubles).  Y is summed from the split-n partials
// of the contraction, in a fixed order, as the right-hand sides are loaded.
// Only the first r_eff rows take part; rows past r_eff of X are written as 0.
//
// XCD-aware launch: workgroups are dispatched to the 8 XCDs round-robin by
// linear index, so workgroup b runs on XCD b % 8; all column groups of unit u
// are given indices with b % 8 == u % 8.  They then share one XCD's L2 and
// walk the same 64-row panels of L at about the same time, so each panel
// comes from HBM about once per unit instead of once per column group.
#include "common.hpp"
#include "weights_layout.hpp"

namespace wc {

// LT[u] = L[u]^T, 32x32 tiles through LDS.
__global__ __launch_bounds__(kBlock) void transpose_l(const double* L, double* LT, int r) {
  __shared__ double tile[32][33];
  const int u = blockIdx.z;
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  const double* Lu = L + (size_t)u * r * r;
  double* LTu = LT + (size_t)u * r * r;
  for (int k = ty; k < 32; k += 8) {
    const int row = by + k, col = bx + tx;
    tile[k][tx] = (row < r && col < r) ? Lu[(size_t)row * r + col] : 0.0;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int row = bx + k, col = by + tx;
    if (row < r && col < r) LTu[(size_t)row * r + col] = tile[tx][k];
  }
}

// A 64x64 block in LDS, XOR-swizzled so that both row-wise (forward) and
// column-wise (backward) lane access are bank-conflict free.
__device__ __forceinline__ int dt_idx(int a, int b) { return a * 64 + (b ^ a); }

// Td <- a 64x64 block (row-major, leading dimension 64) of the inverses;
// each of the NT/64 waves takes 64 / (NT/64) rows.
template <int NT>
__device__ __forceinline__ void stage_inv_block(double* Td, const double* Dt) {
  constexpr int RW = 64 / (NT / 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    const int a = w * RW + q;
    Td[dt_idx(a, lane)] = Dt[a * 64 + lane];
  }
}

// One wave: zq <- B zq for the tile's rows (lane = row), B = the staged
// inverse block (TRANS: its transpose).  The current values go to Zt first
// (one wave's LDS accesses execute in order), then each lane forms its row
// of the product; the solved values are left in Zt for the panel update.
template <int CPW, bool TRANS, int AB>
__device__ __forceinline__ void apply_inv_block(const double* Td, double* Zt, double (&zq)[CPW], int lane, int nt) {
#pragma unroll
  for (int c = 0; c < CPW; ++c) Zt[lane * CPW + c] = lane < nt ? zq[c] : 0.0;
  double acc[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) acc[c] = 0.0;
  // batches of AB k: every LDS read of a batch is issued before its FMAs
  // (same summation order, k = 0 .. 63)
#pragma unroll 1
  for (int k0 = 0; k0 < 64; k0 += AB) {
    double b[AB], zk[AB][CPW];
#pragma unroll
    for (int k = 0; k < AB; ++k) {
      b[k] = TRANS ? Td[dt_idx(k0 + k, lane)] : Td[dt_idx(lane, k0 + k)];
#pragma unroll
      for (int c = 0; c < CPW; ++c) zk[k][c] = Zt[(k0 + k) * CPW + c];
    }
#pragma unroll
    for (int k = 0; k < AB; ++k)
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] = fma(b[k], zk[k][c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    zq[c] = lane < nt ? acc[c] : zq[c];
    Zt[lane * CPW + c] = lane < nt ? acc[c] : 0.0;
  }
}

// Dinv[u][tile] = inverse of the 64x64 diagonal block of L[u] at rows
// 64 tile .. (only the first r_eff rows; the rest of the block is the
// identity).  One wave per block: lane j computes column j of the inverse by
// forward substitution, X[i][j] = (delta_ij - sum_{m<i} L[i][m] X[m][j]) /
// L[i][i], with the block in LDS (row reads are broadcasts) and column j in
// the lane's registers (the loops are unrolled, so every index is constant).
__global__ __launch_bounds__(64) void invert_diag_blocks(const double* L, double* Dinv, const int32_t* r_eff,
                                                         int r) {
  __shared__ double Ls[64 * 64];
  const int tile = blockIdx.x, u = blockIdx.y, j = threadIdx.x;
  const int i0 = tile * 64, re = r_eff[u];
  const int nt = max(0, min(64, re - i0));
  const double* Lu = L + (size_t)u * r * r;
  for (int a = 0; a < 64; ++a)
    Ls[a * 64 + j] = (a < nt && j < nt) ? Lu[(size_t)(i0 + a) * r + i0 + j] : (a == j ? 1.0 : 0.0);
  __syncthreads();
  double x[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    double a0 = i == j ? 1.0 : 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
    for (int m = 0; m + 4 <= i; m += 4) {
      a0 = fma(-Ls[i * 64 + m], x[m], a0);
      a1 = fma(-Ls[i * 64 + m + 1], x[m + 1], a1);
      a2 = fma(-Ls[i * 64 + m + 2], x[m + 2], a2);
      a3 = fma(-Ls[i * 64 + m + 3], x[m + 3], a3);
    }
#pragma unroll
    for (int m = i & ~3; m < i; ++m) a0 = fma(-Ls[i * 64 + m], x[m], a0);
    x[i] = ((a0 + a1) + (a2 + a3)) / Ls[i * 64 + i];
  }
  double* Du = Dinv + ((size_t)u * (r / 64 + 1) + tile) * 64 * 64;
#pragma unroll
  for (int i = 0; i < 64; ++i) Du[i * 64 + j] = x[i];
}

// acc[c] = sum_{j < nt} panel[j * ld] * Zt[j][c], j in order.  A full tile
// loads its 64 panel values in batches of PB, each issued before its FMAs,
// so the loads overlap instead of waiting one after another (PB is bounded
// by the registers a 1024-thread workgroup leaves per lane).
template <int CPW, int PB>
__device__ __forceinline__ void panel_dot(const double* panel, size_t ld, const double* Zt, int nt,
                                          double (&acc)[CPW]) {
#pragma unroll
  for (int c = 0; c < CPW; ++c) acc[c] = 0.0;
  if (nt == 64) {
#pragma unroll 1
    for (int jb = 0; jb < 64; jb += PB) {
      double lv[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) lv[j] = panel[(size_t)(jb + j) * ld];
#pragma unroll
      for (int j = 0; j < PB; ++j)
#pragma unroll
        for (int c = 0; c < CPW; ++c) acc[c] = fma(lv[j], Zt[(jb + j) * CPW + c], acc[c]);
    }
  } else {
    for (int j = 0; j < nt; ++j) {
      const double l = panel[(size_t)j * ld];
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] = fma(l, Zt[j * CPW + c], acc[c]);
    }
  }
}

constexpr int kXcds = 8;
#ifndef WILDCAT_TRSM_XCD
#define WILDCAT_TRSM_XCD 1   // place all column groups of a unit on one XCD
#endif

template <int CPW, int RPT, int NT>
__global__ __launch_bounds__(NT) void trsm_cols(const float* ypart, int nsplit, const double* L,
                                                          const double* LT, const double* Dinv,
                                                          const int32_t* r_eff, float* X, int r,
                                                          int D1, int U, int G) {
  constexpr int kPB = RPT >= 4 ? 8 : 16;   // panel loads per batch
  constexpr int kAB = RPT >= 4 ? 4 : 8;    // inverse-block columns per batch
  __shared__ double Td[64 * 64];
  __shared__ double Zt[64 * CPW];
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = WILDCAT_TRSM_XCD ? (slot / G) * kXcds + xcd : (int)blockIdx.x / G;
  const int c0 = (WILDCAT_TRSM_XCD ? slot % G : (int)blockIdx.x % G) * CPW;
  if (u >= U) return;   // whole workgroup
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int re = r_eff[u];
  const double* Lu = L + (size_t)u * r * r;
  const double* LTu = LT + (size_t)u * r * r;
  const double* Du = Dinv + (size_t)u * (r / 64 + 1) * 64 * 64;

  // Right-hand sides: Y = sum over the contraction's splits, in split order.
  const size_t per_split = (size_t)U * r * D1;
  const float* Yu = ypart + (size_t)u * r * D1;
  double z[RPT][CPW];
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int i = t + q * NT;
#pragma unroll
    for (int c = 0; c < CPW; ++c) z[q][c] = 0.0;
    if (i < re) {
      // 4 splits' loads in flight, then added in split order
      for (int sp0 = 0; sp0 < nsplit; sp0 += 4) {
        float part[4][CPW];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int c = 0; c < CPW; ++c)   // clamped, unconditional loads (no wait behind a branch)
            part[k][c] = Yu[(size_t)min(sp0 + k, nsplit - 1) * per_split + (size_t)i * D1 + min(c0 + c, D1 - 1)];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int c = 0; c < CPW; ++c)
            if (sp0 + k < nsplit && c0 + c < D1) z[q][c] += (double)part[k][c];
      }
    }
  }

  // Forward: L z = y.
  for (int i0 = 0; i0 < re; i0 += 64) {
    const int nt = min(64, re - i0);
    const int qo = i0 / NT, wo = (i0 % NT) / 64;   // owner slot and wave
    stage_inv_block<NT>(Td, Du + (size_t)(i0 / 64) * 64 * 64);
    __syncthreads();
    if (wave == wo) {
      // The owner's rows (slot qo, a uniform branch per slot so that every
      // index stays constant): z_t <- L_tt^{-1} z_t, lane = row.
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        if (q == qo) apply_inv_block<CPW, false, kAB>(Td, Zt, z[q], lane, nt);
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      const int i = t + q * NT;
      if (i >= i0 + nt && i < re) {
        double acc[CPW];
        panel_dot<CPW, kPB>(LTu + (size_t)i0 * r + i, r, Zt, nt, acc);
#pragma unroll
        for (int c = 0; c < CPW; ++c) z[q][c] -= acc[c];
      }
    }
    __syncthreads();
  }

  // Backward: L^T x = z.
  for (int i0 = ((re - 1) / 64) * 64; re > 0 && i0 >= 0; i0 -= 64) {
    const int nt = min(64, re - i0);
    const int qo = i0 / NT, wo = (i0 % NT) / 64;
    stage_inv_block<NT>(Td, Du + (size_t)(i0 / 64) * 64 * 64);
    __syncthreads();
    if (wave == wo) {
      // x_t <- L_tt^{-T} z_t.
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        if (q == qo) apply_inv_block<CPW, true, kAB>(Td, Zt, z[q], lane, nt);
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      const int i = t + q * NT;
      if (i < i0) {
        double acc[CPW];
        panel_dot<CPW, kPB>(Lu + (size_t)i0 * r + i, r, Zt, nt, acc);
#pragma unroll
        for (int c = 0; c < CPW; ++c) z[q][c] -= acc[c];
      }
    }
    __syncthreads();
  }

  float* Xu = X + (size_t)u * r * D1;
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int i = t + q * NT;
    if (i < r) {
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        if (c0 + c < D1) Xu[(size_t)i * D1 + c0 + c] = i < re ? (float)z[q][c] : 0.0f;
    }
  }
}

template <int CPW, int RPT, int NT>
static void launch_trsm_t(int U, int r, int D1, const float* ypart, int nsplit, const double* L, const double* LT,
                          const double* Dinv, const int32_t* r_eff, float* X, hipStream_t st) {
  const int G = (D1 + CPW - 1) / CPW;                      // column groups per unit
  const int slots = (U + kXcds - 1) / kXcds * G;          // workgroups per XCD
  trsm_cols<CPW, RPT, NT><<<slots * kXcds, NT, 0, st>>>(ypart, nsplit, L, LT, Dinv, r_eff, X, r, D1, U, G);
}

// Threads and rows per thread: 256 x 1 up to r = 256, 1024 x 1 up to 1024,
// 1024 x 2 up to 2048, 1024 x 4 up to 4096.
hipError_t launch_trsm(int U, int r, int d, const float* ypart, int nsplit, const double* L, double* LT,
                       double* Dinv, const int32_t* r_eff, float* X, hipStream_t st) {
  const int D1 = d + 1;
  transpose_l<<<dim3((r + 31) / 32, (r + 31) / 32, U), kBlock, 0, st>>>(L, LT, r);
  invert_diag_blocks<<<dim3((r + 63) / 64, U), 64, 0, st>>>(L, Dinv, r_eff, r);
  if (r <= 256) launch_trsm_t<4, 1, 256>(U, r, D1, ypart, nsplit, L, LT, Dinv, r_eff, X, st);
  else if (r <= 1024) launch_trsm_t<4, 1, 1024>(U, r, D1, ypart, nsplit, L, LT, Dinv, r_eff, X, st);
  else if (r <= 2048) launch_trsm_t<4, 2, 1024>(U, r, D1, ypart, nsplit, L, LT, Dinv, r_eff, X, st);
  else launch_trsm_t<4, 4, 1024>(U, r, D1, ypart, nsplit, L, LT, Dinv, r_eff, X, st);
  return hipGetLastError();
}

}  // namespace wc
