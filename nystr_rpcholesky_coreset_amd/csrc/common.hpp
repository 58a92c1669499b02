// Device helpers shared by the WildCat HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wc {

constexpr int kWave = 64;
constexpr int kBlock = 256;          // threads per workgroup for every kernel here
constexpr int kWavesPerBlock = kBlock / kWave;

// bf16 values travel as their 16-bit patterns.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Element loaders: exact float64 / float32 value of an fp32 or bf16 input.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float f32(const float* p, size_t i) { return p[i]; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float f32(const bf16_t* p, size_t i) { return bf16_to_float(p[i].bits); }
};

// Inclusive scan over the 64 lanes of a wave, fixed (Hillis-Steele) order,
// so every caller that scans the same values gets the same bits.
__device__ __forceinline__ double wave_incl_scan(double x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    double y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Workgroup-wide inclusive scan of CNT consecutive values per thread
// (thread t owns elements t*CNT .. t*CNT+CNT-1).  On return v[k] holds the
// inclusive prefix of its element and excl[k] an exclusive prefix: the
// thread's offset for k == 0, else v[k-1] bit for bit.  `total` is the last
// element's inclusive prefix.
// `scratch` needs kWavesPerBlock + 1 doubles of LDS.  Deterministic.
template <int CNT>
__device__ __forceinline__ void block_scan(double (&v)[CNT], double (&excl)[CNT],
                                           double& total, double* scratch) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t / kWave;
#pragma unroll
  for (int k = 1; k < CNT; ++k) v[k] += v[k - 1];
  const double tsum = v[CNT - 1];
  const double incl = wave_incl_scan(tsum);
  double lane_excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) lane_excl = 0.0;
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wave; ++w) off += scratch[w];
  const double base = off + lane_excl;
  double prev = base;
#pragma unroll
  for (int k = 0; k < CNT; ++k) {
    excl[k] = prev;
    v[k] = base + v[k];
    prev = v[k];
  }
  if (t == kBlock - 1) scratch[kWavesPerBlock] = v[CNT - 1];
  __syncthreads();
  total = scratch[kWavesPerBlock];
  __syncthreads();
}

// Workgroup min / max of an int (uses `scratch` ints of LDS, kWavesPerBlock).
__device__ __forceinline__ int block_min_int(int x, int* scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = scratch[0];
  for (int w = 1; w < kWavesPerBlock; ++w) r = min(r, scratch[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_max_int(int x, int* scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = scratch[0];
  for (int w = 1; w < kWavesPerBlock; ++w) r = max(r, scratch[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ double block_sum(double x, double* scratch) {
  x = wave_sum(x);
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = x;
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < kWavesPerBlock; ++w) r += scratch[w];
  __syncthreads();
  return r;
}

__host__ __device__ __forceinline__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace wc
