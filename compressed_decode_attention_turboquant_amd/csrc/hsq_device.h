// Device helpers shared by the libhsq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hsq {

// Work-group barrier for LDS traffic only.  Every hand-over between the waves
// of a work-group goes through LDS, so global loads still in flight (tiles
// prefetched for the next phase) stay in flight across it; __syncthreads()
// would wait for them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Value of v in lane l ^ M (M = 1, 2, 4 or 8; pairs never leave a row of 16
// lanes), over DPP with permutations that are their own inverses, so no
// shift direction is involved: quad permutations for M = 1, 2; for M = 4 the
// quad reversal (l ^ 3) followed by the half-row mirror (l ^ 7); for M = 8 a
// row rotation by 8.  Every lane of the rows involved must be active.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false));
  if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false));
  if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));
  const int r3 = __builtin_amdgcn_update_dpp(0, x, 0x1B, 0xf, 0xf, false);
  return __int_as_float(__builtin_amdgcn_update_dpp(0, r3, 0x141, 0xf, 0xf, false));
}

// One butterfly stage across lanes: the lane without bit M of sub keeps
// v + p, the one with it p - v, both written as p + (+-v) (the same IEEE
// results), so the partner read fuses into the add.
template <int M>
__device__ __forceinline__ void fwht_lane_stage(float (&v)[8], int sub) {
  const uint32_t neg = (sub & M) ? 0x80000000u : 0u;
#pragma unroll
  for (int a = 0; a < 8; ++a) v[a] = xor_lane<M>(v[a]) + __uint_as_float(__float_as_uint(v[a]) ^ neg);
}

// Walsh-Hadamard butterflies (Sylvester order) for a vector spread over LPV
// consecutive lanes (LPV = 8 or 16, aligned in the wave), 8 consecutive
// coordinates per lane: three stages in registers (coordinate bits 0..2),
// then log2(LPV) stages across lanes (coordinate bits 3..).  fp32 throughout.
template <int LPV>
__device__ __forceinline__ void fwht8xlanes(float (&v)[8], int sub) {
  static_assert(LPV == 8 || LPV == 16, "8 or 16 lanes per vector");
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
  fwht_lane_stage<1>(v, sub);
  fwht_lane_stage<2>(v, sub);
  fwht_lane_stage<4>(v, sub);
  if constexpr (LPV == 16) fwht_lane_stage<8>(v, sub);
}

// Sign byte of coordinates [8*sub, 8*sub+8) from a d/32-word mask.
__device__ __forceinline__ uint32_t sign_byte(const uint32_t* mask, int sub) {
  return (mask[sub >> 2] >> (8 * (sub & 3))) & 0xffu;
}

__device__ __forceinline__ float flip(float x, uint32_t bit) {
  return __uint_as_float(__float_as_uint(x) ^ (bit << 31));
}

}  // namespace hsq
