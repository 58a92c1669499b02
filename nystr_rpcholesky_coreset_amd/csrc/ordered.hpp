// Order-preserving integer encoding of float32, for exact min / max
// reductions with integer atomics (min and max are exact and commutative, so
// the result does not depend on the order the atomics land in).
#pragma once

#include <hip/hip_runtime.h>

namespace wc {

// Non-negative floats keep their bits; negative ones have the 31 magnitude
// bits flipped, so signed integer order equals float order (-0 < +0).  The
// map is its own inverse.
__device__ __forceinline__ int ord_enc(float f) {
  const int i = __float_as_int(f);
  return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float ord_dec(int i) { return __int_as_float(i ^ ((i >> 31) & 0x7FFFFFFF)); }

}  // namespace wc
