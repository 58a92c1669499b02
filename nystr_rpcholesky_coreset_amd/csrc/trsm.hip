// Nystroem weights through the pivot block: X = L^{-T} (L^{-1} Y), float64.
//
// [WildCat (arXiv 2602.10056), Nystroem and CompressKV / Alg. 2 paragraphs:
// W = h_tau(K_S, K_S)^{-1} h_tau(K_S, K); with h_tau(K_S, K_S) = L L^T from the
// Cholesky pivot block, W [V, 1] = L^{-T} L^{-1} (h_tau(K_S, K) [V, 1]).]
//
// One wave per (unit, group of CPW right-hand-side columns).  Y is summed from
// the split-n partials of the contraction in a fixed order as it is loaded.
// Rows are processed in tiles of 64 (one row per lane): the part of the sum
// that involves earlier tiles is a per-lane dot product over L's row (forward)
// or column (backward) against the solved values in LDS, and the 64x64
// diagonal block is solved wave-synchronously with shuffles, no barriers.
// Only the first r_eff rows take part; rows past r_eff of X are written as 0.
#include "common.hpp"
#include "layout.hpp"

namespace wc {

template <int CPW>
__global__ __launch_bounds__(kWave) void trsm_cols(const float* ypart, int nsplit, const double* L,
                                                   const int32_t* r_eff, float* X, int U, int r, int D1) {
  extern __shared__ double Z[];   // [r][CPW]
  const int u = blockIdx.y, c0 = blockIdx.x * CPW, lane = threadIdx.x;
  const int re = r_eff[u];
  const double* Lu = L + (size_t)u * r * r;

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
    double v[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) v[c] = 0.0;
    if (lane < nt) {
      const double* Li = Lu + (size_t)i * r;
      double acc[CPW];
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] = 0.0;
      for (int j = 0; j < i0; ++j) {
        const double l = Li[j];
#pragma unroll
        for (int c = 0; c < CPW; ++c) acc[c] = fma(l, Z[j * CPW + c], acc[c]);
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c) v[c] = Z[i * CPW + c] - acc[c];
    }
    for (int k = 0; k < nt; ++k) {
      const double diag = Lu[(size_t)(i0 + k) * r + i0 + k];
      const double lik = (lane > k && lane < nt) ? Lu[(size_t)i * r + i0 + k] : 0.0;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const double zk = __shfl(v[c], k, kWave) / diag;
        if (lane == k) v[c] = zk;
        else if (lane > k && lane < nt) v[c] = fma(-lik, zk, v[c]);
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
    double v[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) v[c] = 0.0;
    if (lane < nt) {
      double acc[CPW];
#pragma unroll
      for (int c = 0; c < CPW; ++c) acc[c] = 0.0;
      for (int j = i0 + nt; j < re; ++j) {
        const double l = Lu[(size_t)j * r + i];
#pragma unroll
        for (int c = 0; c < CPW; ++c) acc[c] = fma(l, Z[j * CPW + c], acc[c]);
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c) v[c] = Z[i * CPW + c] - acc[c];
    }
    for (int k = nt - 1; k >= 0; --k) {
      const double diag = Lu[(size_t)(i0 + k) * r + i0 + k];
      const double lki = (lane < k) ? Lu[(size_t)(i0 + k) * r + i] : 0.0;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const double xk = __shfl(v[c], k, kWave) / diag;
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

hipError_t launch_trsm(int U, int r, int d, const float* ypart, int nsplit, const double* L,
                       const int32_t* r_eff, float* X, hipStream_t st) {
  const int D1 = d + 1;
  if (r <= 2048) {
    constexpr int CPW = 4;
    trsm_cols<CPW><<<dim3((D1 + CPW - 1) / CPW, U), kWave, (size_t)r * CPW * sizeof(double), st>>>(
        ypart, nsplit, L, r_eff, X, U, r, D1);
  } else {
    constexpr int CPW = 2;
    trsm_cols<CPW><<<dim3((D1 + CPW - 1) / CPW, U), kWave, (size_t)r * CPW * sizeof(double), st>>>(
        ypart, nsplit, L, r_eff, X, U, r, D1);
  }
  return hipGetLastError();
}

}  // namespace wc
