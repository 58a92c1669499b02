// Input-range guard: the largest exponent arguments the kernel evaluations
// of a call can meet, from the largest squared row norms of K (and Q).
//
// The library evaluates exp(beta <x, y> / tau^2) without a stabilising
// shift, in fp64 for the selection and in fp32 inside the contractions (the
// pages' exponential kernel taken literally).  By Cauchy-Schwarz every such
// argument is bounded by beta max|k|^2 / tau^2 (four times that with
// recentring: |k - kbar| <= 2 max|k|) for key pairs and by
// beta max|q| max|k| for query/key pairs.  The guard computes both bounds.
#include "common.hpp"

namespace wc {

__global__ __launch_bounds__(64) void range_clear(unsigned long long* m) {
  if (threadIdx.x < 2) m[threadIdx.x] = 0ull;
}

// out <- max(out, max over rows of sum_c x[row][c]^2) in fp64, as the bit
// pattern of a non-negative double (whose unsigned order is the numeric
// order); NaN counts as +inf.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void row_norm_max(const T* X, size_t rows, unsigned long long* out) {
  double mx = 0.0;
  for (size_t row = (size_t)blockIdx.x * kBlock + threadIdx.x; row < rows; row += (size_t)gridDim.x * kBlock) {
    double s = 0.0;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      const double x = (double)Elem<T>::f32(X, row * D + c);
      s = fma(x, x, s);
    }
    if (!(s == s)) s = __builtin_huge_val();
    mx = s > mx ? s : mx;
  }
  __shared__ double part[kBlock / kWave];
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const double o = __shfl_xor(mx, off, kWave);
    mx = o > mx ? o : mx;
  }
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kBlock / kWave; ++w) mx = part[w] > mx ? part[w] : mx;
    atomicMax(out, (unsigned long long)__double_as_longlong(mx));
  }
}

template <typename T>
static void launch_norm_max(int d, const void* X, size_t rows, unsigned long long* out, hipStream_t st) {
  const unsigned grid = (unsigned)((rows + kBlock - 1) / kBlock < 1024 ? (rows + kBlock - 1) / kBlock : 1024);
  const T* p = static_cast<const T*>(X);
  switch (d) {
    case 16: row_norm_max<T, 16><<<grid, kBlock, 0, st>>>(p, rows, out); break;
    case 32: row_norm_max<T, 32><<<grid, kBlock, 0, st>>>(p, rows, out); break;
    case 64: row_norm_max<T, 64><<<grid, kBlock, 0, st>>>(p, rows, out); break;
    case 128: row_norm_max<T, 128><<<grid, kBlock, 0, st>>>(p, rows, out); break;
  }
}

// Host entry used by the C ABI (arguments already validated).  Writes the
// two largest squared norms (keys, queries; 0 without queries) to maxsq and
// synchronises the stream.
hipError_t range_norms(int bf16, int d, const void* K, size_t krows, const void* Q, size_t qrows, double* scratch,
                       double (&maxsq)[2], hipStream_t st) {
  unsigned long long* m = reinterpret_cast<unsigned long long*>(scratch);
  range_clear<<<1, 64, 0, st>>>(m);
  if (bf16) {
    launch_norm_max<bf16_t>(d, K, krows, m, st);
    if (Q) launch_norm_max<bf16_t>(d, Q, qrows, m + 1, st);
  } else {
    launch_norm_max<float>(d, K, krows, m, st);
    if (Q) launch_norm_max<float>(d, Q, qrows, m + 1, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned long long h[2] = {0ull, 0ull};
  if ((e = hipMemcpyAsync(h, m, sizeof(h), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
  maxsq[0] = __builtin_bit_cast(double, h[0]);
  maxsq[1] = __builtin_bit_cast(double, h[1]);
  return hipSuccess;
}

}  // namespace wc
