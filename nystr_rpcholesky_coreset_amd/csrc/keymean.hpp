// Per-unit key mean in float64 (recentring), in two passes so that every
// unit is read by many workgroups at once:
//   key_sum_part   part[u][blk][c] = sum of K[u][l][c] over the rows l of
//                  block blk (kMeanRows rows), in a fixed order;
//   key_mean_final kbar[u][c] = (sum of part[u][blk][c] over blk in order) / n.
// The summation order is fixed, so the result is reproducible bit for bit.
#pragma once

#include "common.hpp"

namespace wc {

constexpr int kMeanRows = 1024;
inline int mean_blocks(int n) { return (n + kMeanRows - 1) / kMeanRows; }

// Thread t sums column t % D over rows l0 + t / D + PH i (PH = 256 / D row
// phases), eight loads in flight into eight partial sums, added pairwise;
// the PH phases meet in LDS and are added in order.
template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void key_sum_part(const TK* K, double* part, int n, int nbk) {
  constexpr int PH = kBlock / D;
  constexpr int ITER = kMeanRows / PH;   // rows per thread
  static_assert(ITER % 8 == 0, "rows per thread");
  __shared__ double s[kBlock];
  const int u = blockIdx.y, blk = blockIdx.x, t = threadIdx.x, c = t % D, ph = t / D;
  const int l0 = blk * kMeanRows;
  const TK* Ku = K + (size_t)u * n * D + c;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
  for (int i0 = 0; i0 < ITER; i0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int l = l0 + ph + PH * (i0 + k);
      v[k] = Elem<TK>::f32(Ku, (size_t)min(l, n - 1) * D);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (l0 + ph + PH * (i0 + k) < n) acc[k] += (double)v[k];
  }
  s[t] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (t < D) {
    double sum = 0.0;
    for (int p = 0; p < PH; ++p) sum += s[p * D + t];
    part[((size_t)u * nbk + blk) * D + t] = sum;
  }
}

template <int D>
__global__ __launch_bounds__(D) void key_mean_final(const double* part, double* kbar, int n, int nbk) {
  const int u = blockIdx.x, c = threadIdx.x;
  double sum = 0.0;
  for (int b = 0; b < nbk; ++b) sum += part[((size_t)u * nbk + b) * D + c];
  kbar[(size_t)u * D + c] = sum / (double)n;
}

template <typename TK, int D>
inline void launch_key_mean(const TK* K, double* part, double* kbar, int U, int n, hipStream_t st) {
  const int nbk = mean_blocks(n);
  key_sum_part<TK, D><<<dim3(nbk, U), kBlock, 0, st>>>(K, part, n, nbk);
  key_mean_final<D><<<U, D, 0, st>>>(part, kbar, n, nbk);
}

}  // namespace wc
