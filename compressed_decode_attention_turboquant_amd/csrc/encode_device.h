// Encoder building blocks shared by the codec kernels and the decode-time
// append kernel (gfx950, wave64): index arithmetic with invariant divisors,
// row loads, and the per-vector norm / rotation / quantisation / packing.
// One vector of d coordinates is spread over d/8 consecutive lanes, 8
// coordinates per lane.
#pragma once

#include "hsq_device.h"
#include "hsq_internal.h"

namespace hsq {
namespace {

// Division of a 32-bit index by a divisor fixed for the launch, with one
// multiply-high, a subtract, an add and two shifts (Granlund and Montgomery,
// "Division by invariant integers using multiplication", PLDI 1994, section 4:
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the quotient
// of every n < 2^32 is (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0), t the
// high word of m n).  Vector indices stay below 2^32 (the entry points
// reject larger counts), so the kernels never divide 64-bit integers.
struct Div32 {
  uint32_t d, m, s1, s2;
};

inline Div32 make_div32(int64_t div) {
  // a divisor the job does not use may be 0; one of 2^32 or more divides
  // every index to 0, as UINT32_MAX does
  const uint32_t d = div < 1 ? 1u : (uint32_t)(div > (int64_t)UINT32_MAX ? UINT32_MAX : div);
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return Div32{d, (uint32_t)m, l < 1 ? l : 1u, l > 1 ? l - 1 : 0u};
}

__device__ __forceinline__ uint32_t udiv(uint32_t n, const Div32& q) {
  const uint32_t t = __umulhi(q.m, n);
  return (t + ((n - t) >> q.s1)) >> q.s2;
}

// vector i -> rotation mask (i / vecs_per_rot) % n_rot
__device__ __forceinline__ uint32_t rot_of(uint32_t i, const Div32& per_rot, const Div32& n_rot) {
  const uint32_t q = udiv(i, per_rot);
  return q - udiv(q, n_rot) * n_rot.d;
}

struct EncodeDivs {
  Div32 unit, seq, rot, nrot, rec;
};

__device__ __forceinline__ int64_t row_of(const EncodeJob& j, const EncodeDivs& q, uint32_t i,
                                          int k) {
  if (j.row_idx) return j.row_idx[(int64_t)i * j.group_n + k];
  if (j.pos) {
    const uint32_t u = udiv(i, q.unit);
    const uint32_t jj = i - u * q.unit.d;
    const uint32_t b = udiv(u, q.seq);
    return (int64_t)u * j.rows_per_unit + j.pos[(int64_t)b * j.pos_per_seq + (int64_t)jj * j.group_n + k];
  }
  return (int64_t)i * j.group_n + k;
}

template <int DT>
__device__ __forceinline__ void load8(const void* x, int64_t off, float (&v)[8]) {
  if constexpr (DT == HSQ_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(ws[k] << 16);
      v[2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
    }
  }
}

// Sum of x over the LPV lanes of a vector (xor butterflies over DPP, no LDS
// round trip).
template <int LPV>
__device__ __forceinline__ float lanes_sum(float x) {
  x += xor_lane<1>(x);
  x += xor_lane<2>(x);
  x += xor_lane<4>(x);
  if constexpr (LPV == 16) x += xor_lane<8>(x);
  return x;
}

// Norm r = ||x|| of the vector whose lanes' sums of squares are ss, and the
// scale inv applied to its unnormalised transform (1 / (r sqrt(d)); 1 / r with
// the rotation off; 0 for the zero vector).  The hardware square root and
// reciprocal (within 1 ulp): every encoder shares this function, so they all
// take the same codes; against the fp64 oracle the differences stay far inside
// the code and norm tolerances.
template <int D, bool ROT>
__device__ __forceinline__ void norm_scale(float ss_lane, float& r, float& inv) {
  constexpr int LPV = D / 8;
  const float ss = lanes_sum<LPV>(ss_lane);
  r = __builtin_amdgcn_sqrtf(ss);
  const float den = ROT ? r * __builtin_sqrtf((float)D) : r;
  inv = r > 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
}

// Quantisation by a bin table.  kSBins equal bins of y * 128 over [-128, 128)
// (unit steps of y * 128, so the bin of a value is the floor of an exactly
// scaled value; values outside go to the end bins); bin b holds the number of
// thresholds below its start and the threshold inside it (times 128, +inf if
// none).  The code of y is that number plus one compare, exact when no bin
// holds two thresholds (true for the Beta codebooks at d = 64 and 128: their
// closest thresholds are >= 0.022 apart, a bin is 1/128 wide).
constexpr int kSBins = 256;
__device__ __forceinline__ void build_sbins(const float* thr, int n_thr, int b, uint2* s_bin,
                                            int* s_two) {
  const float start = (float)(b - kSBins / 2), end = start + 1.f;
  uint32_t below = 0u, inside = 0x7f800000u;
  int n_in = 0;
  for (int h = 0; h < n_thr; ++h) {
    const float t = thr[h] * 128.f;
    below += t < start ? 1u : 0u;
    if (t >= start && t < end) {
      inside = __float_as_uint(t);
      ++n_in;
    }
  }
  s_bin[b] = make_uint2(below, inside);
  if (n_in > 1) *s_two = 1;
}

// Norm, rotation, quantisation and packing of vector i, whose 8 coordinates
// of this lane are in v (LPV lanes per vector).  binned: codes from the bin
// table s_bin (build_sbins); else from the positive thresholds tpos.
template <int D, int BITS, bool ROT>
__device__ __forceinline__ void encode_one(const EncodeJob& j, const EncodeDivs& q, uint32_t i,
                                           int sub, float (&v)[8], uint32_t sword,
                                           const uint32_t (&tpos)[(1 << BITS) / 2 - 1], bool binned,
                                           const uint2* s_bin) {
  constexpr int LPV = D / 8;
  constexpr int L = 1 << BITS;
  constexpr int NPOS = L / 2 - 1;
  const bool valid = i < j.n_vec;
  float ss = 0.f;
#pragma unroll
  for (int a = 0; a < 8; ++a) ss = fmaf(v[a], v[a], ss);
  float r, inv;  // the unnormalised transform scales by sqrt(d)
  norm_scale<D, ROT>(ss, r, inv);

  if constexpr (ROT) {
    const uint32_t sbyte = (sword >> (8 * (sub % 4))) & 0xffu;
#pragma unroll
    for (int a = 0; a < 8; ++a)
      v[a] = __uint_as_float(__float_as_uint(v[a]) ^ (((sbyte >> a) & 1u) << 31));
    fwht8xlanes<LPV>(v, sub);
  }

  uint32_t packed = 0;
  if (binned) {  // work-group uniform
    // y * 128 = v * (inv * 128): scaling by 128 is exact, so this is the
    // rounded y scaled, and its compares with the scaled thresholds are those
    // of y with the thresholds
    const float inv128 = inv * 128.f;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const float y128 = v[a] * inv128;
      const int b = min(max((int)__builtin_floorf(y128), -kSBins / 2), kSBins / 2 - 1) + kSBins / 2;
      const uint2 e = s_bin[b];
      const uint32_t code = e.x + (__uint_as_float(e.y) < y128 ? 1u : 0u);
      packed |= code << (BITS * a);
    }
  } else {
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const float y = v[a] * inv;
      const bool pos = y > 0.f;
      const uint32_t key = (__float_as_uint(y) & 0x7fffffffu) + (pos ? 0u : 1u);
      int cnt = 0;
#pragma unroll
      for (int h = 0; h < NPOS; ++h) cnt += (tpos[h] < key) ? 1 : 0;
      const uint32_t code = pos ? (uint32_t)(L / 2 + cnt) : (uint32_t)(L / 2 - 1 - cnt);
      packed |= code << (BITS * a);
    }
  }

  const uint32_t rec = valid ? udiv(i, q.rec) : 0u;
  const uint32_t slot = i - rec * q.rec.d;
  constexpr int CB = D * BITS / 8;
  uint8_t* crow = j.codes + (int64_t)rec * j.code_rec_bytes + (int64_t)slot * CB;
  if constexpr (BITS == 4) {
    if (valid) reinterpret_cast<uint32_t*>(crow)[sub] = packed;
  } else if constexpr (BITS == 2) {
    // 16 bits per lane; pairs of lanes write one dword
    const uint32_t nxt = __shfl_down(packed, 1, 64);
    if (valid && !(sub & 1)) reinterpret_cast<uint32_t*>(crow)[sub >> 1] = packed | (nxt << 16);
  } else {
    // 24 bits per lane; quads of lanes write three whole dwords.
    const uint32_t nxt = __shfl_down(packed, 1, 64);
    const int qd = sub & 3;
    if (valid && qd < 3)
      reinterpret_cast<uint32_t*>(crow)[3 * (sub >> 2) + qd] = (packed >> (8 * qd)) | (nxt << (24 - 8 * qd));
  }
  if (valid && sub == 0) j.norms[(int64_t)rec * j.norm_rec_floats + slot] = r / (float)j.group_n;
}

}  // namespace
}  // namespace hsq
