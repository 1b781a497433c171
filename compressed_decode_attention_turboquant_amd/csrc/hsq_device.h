// Device helpers shared by the libhsq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hsq {

// Walsh-Hadamard butterflies (Sylvester order) for a vector spread over LPV
// consecutive lanes, 8 consecutive coordinates per lane: three stages in
// registers (coordinate bits 0..2), then log2(LPV) stages across lanes with
// xor shuffles (coordinate bits 3..).  fp32 throughout.
template <int LPV>
__device__ __forceinline__ void fwht8xlanes(float (&v)[8], int sub) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      if (!(a & h)) {
        const float x0 = v[a], x1 = v[a + h];
        v[a] = x0 + x1;
        v[a + h] = x0 - x1;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) {
    const bool upper = (sub & m) != 0;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const float p = __shfl_xor(v[a], m, 64);
      v[a] = upper ? (p - v[a]) : (v[a] + p);
    }
  }
}

// Sign byte of coordinates [8*sub, 8*sub+8) from a d/32-word mask.
__device__ __forceinline__ uint32_t sign_byte(const uint32_t* mask, int sub) {
  return (mask[sub >> 2] >> (8 * (sub & 3))) & 0xffu;
}

__device__ __forceinline__ float flip(float x, uint32_t bit) {
  return __uint_as_float(__float_as_uint(x) ^ (bit << 31));
}

}  // namespace hsq
