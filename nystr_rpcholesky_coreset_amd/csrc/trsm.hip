// Nystroem weights through the pivot block: X = L^{-T} (L^{-1} Y), float64.
//
// [WildCat (arXiv 2602.10056), Nystroem and CompressKV / Alg. 2 paragraphs:
// W = h_tau(K_S, K_S)^{-1} h_tau(K_S, K); with h_tau(K_S, K_S) = L L^T from the
// Cholesky pivot block, W [V, 1] = L^{-T} L^{-1} (h_tau(K_S, K) [V, 1]).]
//
// One wave per (unit, group of CPW right-hand-side columns).  Y is summed from
// the split-n partials of the contraction in a fixed order as it is loaded.
// Rows are processed in tiles of 64 (one row per lane): the part of the sum
// that involves earlier tiles is a per-lane dot product against the solved
// values in LDS (broadcast reads), and the 64x64 diagonal block is solved
// wave-synchronously with shuffles, no barriers.  The forward sweep reads
// L^T (a transposed copy made first) and the backward sweep reads L, so at
// every step the 64 lanes read 64 consecutive doubles of one row.  Only the
// first r_eff rows take part; rows past r_eff of X are written as 0.
#include "common.hpp"
#include "layout.hpp"

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

// Diagonal 64x64 tile of L in LDS, XOR-swizzled so that both row-wise
// (forward) and column-wise (backward) lane access are bank-conflict free.
__device__ __forceinline__ int dt_idx(int a, int b) { return a * 64 + (b ^ a); }

// Td <- L[i0 .. i0+nt)[i0 .. i0+nt) (zeros outside), 16 rows in flight.
__device__ __forceinline__ void stage_diag(double* Td, const double* Lu, int r, int i0, int nt, int lane) {
  for (int a0 = 0; a0 < 64; a0 += 16) {
    double x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int a = a0 + q;
      x[q] = (a < nt && lane < nt) ? Lu[(size_t)(i0 + a) * r + i0 + lane] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) Td[dt_idx(a0 + q, lane)] = x[q];
  }
  __syncthreads();
}

template <int CPW>
__global__ __launch_bounds__(kWave) void trsm_cols(const float* ypart, int nsplit, const double* L, const double* LT,
                                                   const int32_t* r_eff, float* X, int U, int r, int D1) {
  extern __shared__ double smem[];
  double* Z = smem;                        // [r][CPW]
  double* Td = smem + (size_t)r * CPW;     // [64][64] swizzled diagonal tile
  const int u = blockIdx.y, c0 = blockIdx.x * CPW, lane = threadIdx.x;
  const int re = r_eff[u];
  const double* Lu = L + (size_t)u * r * r;
  const double* LTu = LT + (size_t)u * r * r;

  for (int i = lane; i < re; i += kWave) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      double acc = 0.0;
      if (c0 + c < D1)
        for (int s = 0; s < nsplit; ++s) acc += (double)ypart[(((size_t)s * U + u) * r + i) * D1 + c0 + c];
      Z[i * CPW + c] = acc;
    }
  }
  __syncthreads();

  // Forward: L z = y.
  for (int i0 = 0; i0 < re; i0 += kWave) {
    const int nt = min(kWave, re - i0);
    const int i = i0 + lane;
    stage_diag(Td, Lu, r, i0, nt, lane);
    const double inv = lane < nt ? 1.0 / Td[dt_idx(lane, lane)] : 0.0;
    double v[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) v[c] = 0.0;
    if (lane < nt) {
      double acc[CPW];
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] = 0.0;
#pragma unroll 16
      for (int j = 0; j < i0; ++j) {
        const double l = LTu[(size_t)j * r + i];
#pragma unroll
        for (int c = 0; c < CPW; ++c) acc[c] = fma(l, Z[j * CPW + c], acc[c]);
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c) v[c] = Z[i * CPW + c] - acc[c];
    }
    for (int k = 0; k < nt; ++k) {
      const double ik = __shfl(inv, k, kWave);
      const double lik = (lane > k && lane < nt) ? Td[dt_idx(lane, k)] : 0.0;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const double zk = __shfl(v[c], k, kWave) * ik;
        if (lane == k) v[c] = zk;
        else if (lane > k) v[c] = fma(-lik, zk, v[c]);
      }
    }
    if (lane < nt) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) Z[i * CPW + c] = v[c];
    }
    __syncthreads();
  }

  // Backward: L^T x = z.
  for (int i0 = ((re - 1) / kWave) * kWave; re > 0 && i0 >= 0; i0 -= kWave) {
    const int nt = min(kWave, re - i0);
    const int i = i0 + lane;
    stage_diag(Td, Lu, r, i0, nt, lane);
    const double inv = lane < nt ? 1.0 / Td[dt_idx(lane, lane)] : 0.0;
    double v[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) v[c] = 0.0;
    if (lane < nt) {
      double acc[CPW];
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] = 0.0;
#pragma unroll 16
      for (int j = i0 + nt; j < re; ++j) {
        const double l = Lu[(size_t)j * r + i];
#pragma unroll
        for (int c = 0; c < CPW; ++c) acc[c] = fma(l, Z[j * CPW + c], acc[c]);
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c) v[c] = Z[i * CPW + c] - acc[c];
    }
    for (int k = nt - 1; k >= 0; --k) {
      const double ik = __shfl(inv, k, kWave);
      const double lki = (lane < k) ? Td[dt_idx(k, lane)] : 0.0;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const double xk = __shfl(v[c], k, kWave) * ik;
        if (lane == k) v[c] = xk;
        else if (lane < k) v[c] = fma(-lki, xk, v[c]);
      }
    }
    if (lane < nt) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) Z[i * CPW + c] = v[c];
    }
    __syncthreads();
  }

  float* Xu = X + (size_t)u * r * D1;
  for (int i = lane; i < r; i += kWave) {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (c0 + c < D1) Xu[(size_t)i * D1 + c0 + c] = i < re ? (float)Z[i * CPW + c] : 0.0f;
  }
}

template <int CPW>
static void launch_trsm_cpw(int U, int r, int D1, const float* ypart, int nsplit, const double* L, const double* LT,
                            const int32_t* r_eff, float* X, hipStream_t st) {
  const size_t lds = ((size_t)r * CPW + 64 * 64) * sizeof(double);
  trsm_cols<CPW><<<dim3((D1 + CPW - 1) / CPW, U), kWave, lds, st>>>(ypart, nsplit, L, LT, r_eff, X, U, r, D1);
}

// Columns per wave chosen so that the solved values plus the diagonal tile
// fit in 64 KiB of LDS: 4 up to r = 1024, 2 up to 2048, 1 up to 4096.
hipError_t launch_trsm(int U, int r, int d, const float* ypart, int nsplit, const double* L, double* LT,
                       const int32_t* r_eff, float* X, hipStream_t st) {
  const int D1 = d + 1;
  transpose_l<<<dim3((r + 31) / 32, (r + 31) / 32, U), kBlock, 0, st>>>(L, LT, r);
  if (r <= 1024) launch_trsm_cpw<4>(U, r, D1, ypart, nsplit, L, LT, r_eff, X, st);
  else if (r <= 2048) launch_trsm_cpw<2>(U, r, D1, ypart, nsplit, L, LT, r_eff, X, st);
  else launch_trsm_cpw<1>(U, r, D1, ypart, nsplit, L, LT, r_eff, X, st);
  return hipGetLastError();
}

}  // namespace wc
