// TurboQuant encode / decode kernels for gfx950.
//
// [Tamarin (HSQ) summary, section 2, "Key technical components",
// quantisation: scalar quantisation after a fixed random orthonormal
// rotation; Ablation, Statistical Inference, and Validation for KV-Cache
// Compression, technical summary, "Experimental setup": random
// Walsh-Hadamard transform, then a Beta Lloyd-Max codebook.]
//
// One vector of d coordinates is spread over d/8 lanes, 8 consecutive
// coordinates per lane (d=128: 16 lanes, 4 vectors per wave64).  The
// Walsh-Hadamard transform runs three butterfly stages inside each lane's
// registers and log2(d/8) stages across lanes with xor shuffles, all in fp32.
// Quantisation counts thresholds with the codebook's odd symmetry: only the
// 2^(b-1)-1 positive thresholds are compared, against |y| as integer bit
// patterns (for non-negative floats the bit order is the numeric order), with
// a +1 on the key for y <= 0 to turn "t < y" into "t <= |y|".
//
// Variants [Ablation ..., "Key contributions" item 1 and "Results and
// recommendations"]: ROT = false is Plain-KV, the same steps with the
// rotation off (y = x / r); BITS = 2 packs four codes per byte in the same
// LSB-first order as the 3-bit stream.
#include "encode_device.h"

namespace hsq {
namespace {

constexpr int kWG = 256;
constexpr int kVPT = 2;  // vectors per thread in the encoder
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// CONTIG: one row per vector, row i (group_n == 1, no row_idx, no pos); the
// loads are then straight-line, at indices clamped into the array, so that
// no wait sits between them.
template <int D, int BITS, int DT, bool ROT, bool CONTIG>
__global__ __launch_bounds__(kWG) void encode_kernel(EncodeJob j, EncodeDivs q) {
  constexpr int LPV = D / 8;
  constexpr int VPB = kWG / LPV;  // vectors per pass of the work-group
  constexpr int L = 1 << BITS;
  constexpr int NPOS = L / 2 - 1;  // positive thresholds t[L/2 .. L-2]
  const int sub = threadIdx.x % LPV;
  const uint32_t i0 = blockIdx.x * (kVPT * VPB) + threadIdx.x / LPV;

  // Global loads first: the thresholds, then every vector of this thread
  // (i0 + u VPB) with its sign word, all in flight together.
  uint32_t tpos[NPOS];
#pragma unroll
  for (int h = 0; h < NPOS; ++h) tpos[h] = __float_as_uint(j.thr[L / 2 + h]);
  uint32_t sword[kVPT];
  float v[kVPT][8];
#pragma unroll
  for (int u = 0; u < kVPT; ++u) {
    const uint32_t i = i0 + u * VPB;
    const bool valid = i < j.n_vec;
    const uint32_t ic = valid ? i : (uint32_t)(j.n_vec - 1);  // past the end: reread the last
    sword[u] = 0u;
    if constexpr (ROT) sword[u] = j.signs[rot_of(ic, q.rot, q.nrot) * (D / 32) + sub / 4];
    if constexpr (CONTIG) {
      load8<DT>(j.x, (int64_t)ic * D + 8 * sub, v[u]);
    } else {
#pragma unroll
      for (int a = 0; a < 8; ++a) v[u][a] = 0.f;
      if (valid) {
        for (int k = 0; k < j.group_n; ++k) {
          float t[8];
          load8<DT>(j.x, row_of(j, q, i, k) * D + 8 * sub, t);
#pragma unroll
          for (int a = 0; a < 8; ++a) v[u][a] += t[a];
        }
      }
    }
  }

  // the bin table of the quantiser, built while the loads above are in
  // flight; a codebook with two thresholds in one bin falls back to counting
  // the thresholds (work-group uniform)
  static_assert(kWG == kSBins, "one bin per thread");
  __shared__ uint2 s_bin[kSBins];
  __shared__ int s_two;
  if (threadIdx.x == 0) s_two = 0;
  lds_barrier();
  build_sbins(j.thr, L - 1, threadIdx.x, s_bin, &s_two);
  lds_barrier();
  const bool binned = s_two == 0;

#pragma unroll
  for (int u = 0; u < kVPT; ++u)
    encode_one<D, BITS, ROT>(j, q, i0 + u * VPB, sub, v[u], sword[u], tpos, binned, s_bin);
}

// Code table of the decoder: one entry per byte of codes (BITS = 4: two
// centroids, BITS = 2: four) or per 6-bit field (BITS = 3: two), so one LDS
// read dequantises 2 or 4 coordinates.
template <int BITS>
struct DecTab {
  static constexpr int kEntries = BITS == 3 ? 64 : 256;
  static constexpr int kPer = BITS == 2 ? 4 : 2;  // coordinates per entry
};

constexpr int kDecVPT = 4;  // vectors per thread in the decoder, loads issued together

// RoPE turns per position of each coordinate pair f < d/2, base^(-2f/d) /
// (2 pi), as a 64-bit binary fraction (low and high words), so that the
// fraction of a turn at any int32 position is one wrapping integer product.
// Written by threads 0 .. d/2 - 1 of the work-group.
template <int D>
__device__ __forceinline__ void rope_turns(double base, uint32_t* lo, uint32_t* hi) {
  if (threadIdx.x < D / 2) {
    const double t = pow(base, -2.0 * threadIdx.x / D) * (0.5 / 3.141592653589793);
    const uint64_t fx = (uint64_t)((t - __builtin_floor(t)) * 0x1p64);
    lo[threadIdx.x] = (uint32_t)fx;
    hi[threadIdx.x] = (uint32_t)(fx >> 32);
  }
}
template <int D, int BITS, int OUT, bool ROT>
__global__ __launch_bounds__(kWG) void decode_kernel(DecodeJob j, Div32 per_rot, Div32 n_rot) {
  constexpr int LPV = D / 8;
  constexpr int VPB = kWG / LPV;
  constexpr int U = kDecVPT;
  constexpr int CB = D * BITS / 8;
  constexpr int CW = BITS == 3 ? 2 : 1;  // code dwords loaded per lane and vector
  constexpr int NE = DecTab<BITS>::kEntries, PER = DecTab<BITS>::kPer;
  __shared__ __align__(16) float tab[NE * PER];
  if (threadIdx.x < NE) {
    constexpr uint32_t M = (1u << BITS) - 1;
#pragma unroll
    for (int k = 0; k < PER; ++k)
      tab[threadIdx.x * PER + k] = j.centroids[(threadIdx.x >> (BITS * k)) & M];
  }
  __syncthreads();
  const int sub = threadIdx.x % LPV;
  // This lane's code bits of a row: BITS = 4 one dword; 2: half a dword;
  // 3: 24 bits from bit 24 sub (two dwords, the second inside the row).
  const int bit = BITS * 8 * sub;
  const int w0 = bit >> 5, sh = bit & 31;
  const int w1 = min(w0 + 1, CB / 4 - 1);
  // Blocks of U * VPB vectors, one per work-group; every load of a block
  // (codes, norm, sign word) is issued before the first vector is decoded.
  const uint64_t nblk = ((uint64_t)j.n_vec + U * VPB - 1) / (U * VPB);
  for (uint64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    uint32_t cw[U][CW];
    float r[U];
    uint32_t sw[U];
    bool valid[U];
    uint32_t idx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t i64 = blk * (U * VPB) + (uint64_t)(u * VPB) + threadIdx.x / LPV;
      valid[u] = i64 < (uint64_t)j.n_vec;
      const uint32_t i = valid[u] ? (uint32_t)i64 : (uint32_t)(j.n_vec - 1);  // reread the last
      idx[u] = i;
      const uint32_t* row = reinterpret_cast<const uint32_t*>(j.codes + (int64_t)i * CB);
      cw[u][0] = row[w0];
      if constexpr (CW == 2) cw[u][1] = row[w1];
      r[u] = j.norms[i];
      sw[u] = 0u;
      if constexpr (ROT) sw[u] = j.signs[rot_of(i, per_rot, n_rot) * (D / 32) + sub / 4];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t codes;
      if constexpr (BITS == 4) {
        codes = cw[u][0];
      } else if constexpr (BITS == 2) {
        codes = cw[u][0] >> sh;
      } else {
        codes = (uint32_t)(((uint64_t)cw[u][1] << 32 | cw[u][0]) >> sh);
      }
      float v[8];
      if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 c = reinterpret_cast<const float2*>(tab)[(codes >> (8 * k)) & 0xffu];
          v[2 * k] = c.x;
          v[2 * k + 1] = c.y;
        }
      } else if constexpr (BITS == 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float4 c = reinterpret_cast<const float4*>(tab)[(codes >> (8 * k)) & 0xffu];
          v[4 * k] = c.x;
          v[4 * k + 1] = c.y;
          v[4 * k + 2] = c.z;
          v[4 * k + 3] = c.w;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 c = reinterpret_cast<const float2*>(tab)[(codes >> (6 * k)) & 63u];
          v[2 * k] = c.x;
          v[2 * k + 1] = c.y;
        }
      }
      if constexpr (ROT) fwht8xlanes<LPV>(v, sub);
      // 1 / sqrt(d) is a compile-time constant: one multiply, not a division
      const float s = ROT ? r[u] * (1.f / __builtin_sqrtf((float)D)) : r[u];
      const uint32_t sbyte = ROT ? (sw[u] >> (8 * (sub % 4))) & 0xffu : 0u;
#pragma unroll
      for (int a = 0; a < 8; ++a)
        v[a] = __uint_as_float(__float_as_uint(v[a] * s) ^ (((sbyte >> a) & 1u) << 31));
      if (valid[u]) {
        const uint32_t i = idx[u];
        if constexpr (OUT == HSQ_F32) {
          float4* o = reinterpret_cast<float4*>(static_cast<float*>(j.out) + (int64_t)i * D + 8 * sub);
          o[0] = make_float4(v[0], v[1], v[2], v[3]);
          o[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          // round to nearest even, two values per conversion instruction
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            w[k] = __builtin_bit_cast(uint32_t,
                                      __builtin_convertvector(f32x2{v[2 * k], v[2 * k + 1]}, bf16x2));
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(j.out) + (int64_t)i * D + 8 * sub) =
              make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  }
}

template <int D, int BITS, bool ROT>
hipError_t encode_dt(const EncodeJob& j, hipStream_t s) {
  constexpr int VPB = kVPT * kWG / (D / 8);
  const int64_t grid = (j.n_vec + VPB - 1) / VPB;
  const EncodeDivs q{make_div32(j.vecs_per_unit), make_div32(j.units_per_seq),
                     make_div32(j.vecs_per_rot), make_div32(j.n_rot), make_div32(j.vecs_per_rec)};
  const bool contig = j.group_n == 1 && !j.row_idx && !j.pos;
  const dim3 g((unsigned)grid), b(kWG);
  if (j.dtype == HSQ_F32) {
    if (contig)
      hipLaunchKernelGGL((encode_kernel<D, BITS, HSQ_F32, ROT, true>), g, b, 0, s, j, q);
    else
      hipLaunchKernelGGL((encode_kernel<D, BITS, HSQ_F32, ROT, false>), g, b, 0, s, j, q);
  } else {
    if (contig)
      hipLaunchKernelGGL((encode_kernel<D, BITS, HSQ_BF16, ROT, true>), g, b, 0, s, j, q);
    else
      hipLaunchKernelGGL((encode_kernel<D, BITS, HSQ_BF16, ROT, false>), g, b, 0, s, j, q);
  }
  return hipGetLastError();
}

// Fetched keys of a pre-RoPE archive (RopeKeysJob): one vector per D/8
// lanes, kDecVPT vectors per lane group with their loads issued together
// (each vector's address waits on its selection entry), in blocks strided
// over a grid of at most the resident work-groups (the turns table costs a
// set-up per work-group).  Lane sub of a vector holds coordinates
// 4 sub .. 4 sub + 3 (registers 0-3) and D/2 + 4 sub .. (registers 4-7), so
// every rotary pair (f, f + D/2) sits in one lane and the rotation needs no
// partner lane.  The transform back to the model's domain does not care
// which coordinate bit a lane or register bit stands for (the Hadamard
// matrix is the same under a permutation of the index bits applied to rows
// and columns): register bits 0, 1, 2 are coordinate bits 0, 1 and
// log2(D) - 1, lane bits are coordinate bits 2 .. log2(D) - 2.  A slot whose
// selection names no group gets a zero row.  Indices past the end are
// clamped to the last vector (recomputed, not stored), so every lane runs
// the cross-lane steps.
template <int D>
__global__ __launch_bounds__(kWG) void rope_keys_kernel(RopeKeysJob j) {
  constexpr int LPV = D / 8, VPB = kWG / LPV, CB = D / 2, U = kDecVPT, H = D / 2;
  __shared__ __align__(16) float tab[256 * 2];  // code byte -> its two centroids
  __shared__ uint32_t turns_lo[D / 2], turns_hi[D / 2];
  if (threadIdx.x < 256) {
    tab[2 * threadIdx.x] = j.cb4[threadIdx.x & 15];
    tab[2 * threadIdx.x + 1] = j.cb4[threadIdx.x >> 4];
  }
  rope_turns<D>(j.rope_base, turns_lo, turns_hi);
  __syncthreads();
  const int sub = threadIdx.x % LPV;
  // this lane's four pair angles: f = 4 sub + k
  uint32_t tlo[4], thi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    tlo[k] = turns_lo[4 * sub + k];
    thi[k] = turns_hi[4 * sub + k];
  }
  const uint32_t N = (uint32_t)j.group_n, beta = (uint32_t)j.beta, Hkv = (uint32_t)j.Hkv;
  const uint64_t rec = (uint64_t)N * (D + 8);
  const uint32_t n_vec = (uint32_t)j.units * beta * N;  // < 2^31 (launch_rope_keys)
  const uint32_t nblk = (n_vec + VPB * U - 1) / (VPB * U);
  const float isd = 1.f / __builtin_sqrtf((float)D);
  for (uint32_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    uint32_t i[U];
    bool valid[U], ok[U];
    uint32_t clo[U], chi[U], sbyte[U];
    int32_t p[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint32_t i0 = (blk * U + k) * VPB + threadIdx.x / LPV;
      valid[k] = i0 < n_vec;
      i[k] = valid[k] ? i0 : n_vec - 1;
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      // 32-bit quotients (a 64-bit division is a long software sequence)
      const uint32_t us = i[k] / N, t = i[k] - us * N;  // us = u * beta + s
      const uint32_t u = us / beta, b = u / Hkv, h = u - b * Hkv;
      const int g0 = j.idx[us];
      ok[k] = g0 >= 0 && g0 < j.n_groups;
      const uint32_t g = ok[k] ? (uint32_t)g0 : 0u;
      // the record: in place by group, or gathered by slot (staged)
      const uint64_t r = j.staged ? (uint64_t)us : (uint64_t)u * j.unit_recs + g;
      const uint8_t* row = j.l3 + r * rec + t * CB;
      // codes of coordinates 4 sub .. +3 and H + 4 sub .. +3 (two bytes each)
      clo[k] = *reinterpret_cast<const uint16_t*>(row + 2 * sub);
      chi[k] = *reinterpret_cast<const uint16_t*>(row + H / 2 + 2 * sub);
      p[k] = j.group_pos[(uint64_t)b * j.pos_per_seq + g * N + t];
      const uint32_t* m = j.k_signs + h * (D / 32);
      const int c0 = 4 * sub, c1 = H + 4 * sub;
      sbyte[k] = ((m[c0 >> 5] >> (c0 & 31)) & 0xfu) | (((m[c1 >> 5] >> (c1 & 31)) & 0xfu) << 4);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float2 e0 = reinterpret_cast<const float2*>(tab)[(clo[k] >> (8 * c)) & 0xffu];
        const float2 e1 = reinterpret_cast<const float2*>(tab)[(chi[k] >> (8 * c)) & 0xffu];
        v[2 * c] = e0.x;
        v[2 * c + 1] = e0.y;
        v[4 + 2 * c] = e1.x;
        v[4 + 2 * c + 1] = e1.y;
      }
      // back to the model's domain: x = D H c / sqrt(d)
      fwht8xlanes<LPV>(v, sub);
#pragma unroll
      for (int a = 0; a < 8; ++a) v[a] = flip(v[a] * isd, (sbyte[k] >> a) & 1u);
      // RoPE on the lane's four pairs (v[a], v[a + 4]), angle p * turns[4 sub + a]
      const uint32_t pu = (uint32_t)p[k];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        // top word of p * turns mod 2^64 (a negative p is pu - 2^32)
        const uint32_t top = __umulhi(pu, tlo[a]) + pu * thi[a] - (p[k] < 0 ? tlo[a] : 0u);
        const float rev = (float)top * 0x1p-32f;
        const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
        const float x0 = v[a], x1 = v[a + 4];
        v[a] = x0 * cs - x1 * sn;
        v[a + 4] = x1 * cs + x0 * sn;
      }
      uint32_t w[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const _Float16 lo = ok[k] ? (_Float16)v[2 * c] : (_Float16)0.f;
        const _Float16 hi = ok[k] ? (_Float16)v[2 * c + 1] : (_Float16)0.f;
        w[c] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      if (valid[k]) {
        uint16_t* o = j.out + (uint64_t)i[k] * D;
        *reinterpret_cast<uint2*>(o + 4 * sub) = make_uint2(w[0], w[1]);
        *reinterpret_cast<uint2*>(o + H + 4 * sub) = make_uint2(w[2], w[3]);
      }
    }
  }
}

// RoPE fetch (hsq_decode_rope) with each rotary pair in one lane: lane sub
// holds coordinates 4 sub .. 4 sub + 3 (registers 0-3) and D/2 + 4 sub ..
// (registers 4-7), as in rope_keys_kernel, so the rotation needs no partner
// lane; the in-register FWHT runs unchanged under that relabelling of the
// coordinate bits.  kDecVPT vectors per lane group with all their loads
// issued first; at most a chip of resident work-groups striding over the
// blocks (the turns table costs a set-up per work-group).
template <int D, int BITS, int OUT, bool ROT>
__global__ __launch_bounds__(kWG) void rope_decode_kernel(DecodeJob j, Div32 per_rot,
                                                          Div32 n_rot) {
  constexpr int LPV = D / 8, VPB = kWG / LPV, U = kDecVPT, H = D / 2;
  constexpr int CB = D * BITS / 8;
  constexpr int NE = DecTab<BITS>::kEntries, PER = DecTab<BITS>::kPer;
  constexpr int FB = BITS * PER;  // code bits per table entry
  __shared__ __align__(16) float tab[NE * PER];
  __shared__ uint32_t turns_lo[D / 2], turns_hi[D / 2];
  if (threadIdx.x < NE) {
    constexpr uint32_t M = (1u << BITS) - 1;
#pragma unroll
    for (int k = 0; k < PER; ++k)
      tab[threadIdx.x * PER + k] = j.centroids[(threadIdx.x >> (BITS * k)) & M];
  }
  rope_turns<D>(j.rope_base, turns_lo, turns_hi);
  __syncthreads();
  const int sub = threadIdx.x % LPV;
  uint32_t tlo[4], thi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    tlo[k] = turns_lo[4 * sub + k];
    thi[k] = turns_hi[4 * sub + k];
  }
  // the 4 * BITS code bits of coordinates c .. c + 3 of a row (byte loads:
  // 3-bit fields start on half bytes)
  auto codes4 = [&](const uint8_t* row, int c) -> uint32_t {
    const int bit = BITS * c, b0 = bit >> 3;
    uint32_t w = row[b0];
    if constexpr (BITS > 2) w |= (uint32_t)row[b0 + 1] << 8;
    return (w >> (bit & 7)) & ((1u << (4 * BITS)) - 1u);
  };
  const uint64_t nblk = ((uint64_t)j.n_vec + U * VPB - 1) / (U * VPB);
  for (uint64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    uint32_t clo[U], chi[U], sbyte[U], idx[U];
    float r[U];
    int32_t ps[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t i64 = blk * (U * VPB) + (uint64_t)(u * VPB) + threadIdx.x / LPV;
      valid[u] = i64 < (uint64_t)j.n_vec;
      const uint32_t i = valid[u] ? (uint32_t)i64 : (uint32_t)(j.n_vec - 1);  // reread the last
      idx[u] = i;
      const uint8_t* row = j.codes + (int64_t)i * CB;
      clo[u] = codes4(row, 4 * sub);
      chi[u] = codes4(row, H + 4 * sub);
      r[u] = j.norms[i];
      sbyte[u] = 0u;
      if constexpr (ROT) {
        const uint32_t* m = j.signs + rot_of(i, per_rot, n_rot) * (D / 32);
        const int c0 = 4 * sub, c1 = H + 4 * sub;
        sbyte[u] = ((m[c0 >> 5] >> (c0 & 31)) & 0xfu) | (((m[c1 >> 5] >> (c1 & 31)) & 0xfu) << 4);
      }
      ps[u] = j.pos[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 4 / PER; ++e) {
        const float* t0 = tab + ((clo[u] >> (FB * e)) & (NE - 1)) * PER;
        const float* t1 = tab + ((chi[u] >> (FB * e)) & (NE - 1)) * PER;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          v[PER * e + k] = t0[k];
          v[4 + PER * e + k] = t1[k];
        }
      }
      if constexpr (ROT) fwht8xlanes<LPV>(v, sub);
      const float sc = ROT ? r[u] * (1.f / __builtin_sqrtf((float)D)) : r[u];
#pragma unroll
      for (int a = 0; a < 8; ++a) v[a] = flip(v[a] * sc, (sbyte[u] >> a) & 1u);
      const uint32_t pu = (uint32_t)ps[u];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        // top word of p * turns mod 2^64 (a negative p is pu - 2^32)
        const uint32_t top = __umulhi(pu, tlo[a]) + pu * thi[a] - (ps[u] < 0 ? tlo[a] : 0u);
        const float rev = (float)top * 0x1p-32f;
        const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
        const float x0 = v[a], x1 = v[a + 4];
        v[a] = x0 * cs - x1 * sn;
        v[a + 4] = x1 * cs + x0 * sn;
      }
      if (valid[u]) {
        const int64_t o = (int64_t)idx[u] * D;
        if constexpr (OUT == HSQ_F32) {
          float* dst = static_cast<float*>(j.out) + o;
          *reinterpret_cast<float4*>(dst + 4 * sub) = make_float4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<float4*>(dst + H + 4 * sub) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            w[k] = __builtin_bit_cast(uint32_t,
                                      __builtin_convertvector(f32x2{v[2 * k], v[2 * k + 1]}, bf16x2));
          uint16_t* dst = static_cast<uint16_t*>(j.out) + o;
          *reinterpret_cast<uint2*>(dst + 4 * sub) = make_uint2(w[0], w[1]);
          *reinterpret_cast<uint2*>(dst + H + 4 * sub) = make_uint2(w[2], w[3]);
        }
      }
    }
  }
}

template <int D, int BITS, bool ROT, bool ROPE>
hipError_t decode_out(const DecodeJob& j, hipStream_t s) {
  constexpr int VPB = kWG / (D / 8);
  // the RoPE variant: at most a chip of resident work-groups (256 CUs, 4
  // work-groups of 4 waves each), each striding over the blocks
  const int64_t blocks = (j.n_vec + kDecVPT * VPB - 1) / (kDecVPT * VPB);
  const int64_t grid = ROPE ? std::min<int64_t>(blocks, 256 * 4) : blocks;
  const Div32 per_rot = make_div32(j.vecs_per_rot), n_rot = make_div32(j.n_rot);
  if constexpr (ROPE) {
    if (j.out_dtype == HSQ_F32)
      hipLaunchKernelGGL((rope_decode_kernel<D, BITS, HSQ_F32, ROT>), dim3((unsigned)grid),
                         dim3(kWG), 0, s, j, per_rot, n_rot);
    else
      hipLaunchKernelGGL((rope_decode_kernel<D, BITS, HSQ_BF16, ROT>), dim3((unsigned)grid),
                         dim3(kWG), 0, s, j, per_rot, n_rot);
  } else {
    if (j.out_dtype == HSQ_F32)
      hipLaunchKernelGGL((decode_kernel<D, BITS, HSQ_F32, ROT>), dim3((unsigned)grid), dim3(kWG),
                         0, s, j, per_rot, n_rot);
    else
      hipLaunchKernelGGL((decode_kernel<D, BITS, HSQ_BF16, ROT>), dim3((unsigned)grid), dim3(kWG),
                         0, s, j, per_rot, n_rot);
  }
  return hipGetLastError();
}

template <int D, int BITS, bool ROT>
hipError_t decode_dt(const DecodeJob& j, hipStream_t s) {
  return j.pos ? decode_out<D, BITS, ROT, true>(j, s) : decode_out<D, BITS, ROT, false>(j, s);
}

template <int D, bool ROT>
hipError_t encode_bits(const EncodeJob& j, hipStream_t s) {
  if (j.bits == 4) return encode_dt<D, 4, ROT>(j, s);
  if (j.bits == 3) return encode_dt<D, 3, ROT>(j, s);
  return encode_dt<D, 2, ROT>(j, s);
}

template <int D, bool ROT>
hipError_t decode_bits(const DecodeJob& j, hipStream_t s) {
  if (j.bits == 4) return decode_dt<D, 4, ROT>(j, s);
  if (j.bits == 3) return decode_dt<D, 3, ROT>(j, s);
  return decode_dt<D, 2, ROT>(j, s);
}

}  // namespace

// signs == nullptr selects the rotation-off variant
hipError_t launch_encode(const EncodeJob& j, hipStream_t s) {
  if (j.n_vec <= 0) return hipSuccess;
  if (j.n_vec > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  const bool rot = j.signs != nullptr;
  if (j.d == 128) return rot ? encode_bits<128, true>(j, s) : encode_bits<128, false>(j, s);
  return rot ? encode_bits<64, true>(j, s) : encode_bits<64, false>(j, s);
}

hipError_t launch_rope_keys(const RopeKeysJob& j, hipStream_t s) {
  const int64_t n_vec = (int64_t)j.units * j.beta * j.group_n;
  if (n_vec <= 0) return hipSuccess;
  if (n_vec >= (int64_t(1) << 31)) return hipErrorInvalidValue;  // 32-bit vector index
  const int64_t vpb = kWG / (j.d / 8) * kDecVPT;
  const int64_t grid = std::min<int64_t>((n_vec + vpb - 1) / vpb, 256 * 4);
  if (j.d == 128)
    hipLaunchKernelGGL(rope_keys_kernel<128>, dim3((unsigned)grid), dim3(kWG), 0, s, j);
  else
    hipLaunchKernelGGL(rope_keys_kernel<64>, dim3((unsigned)grid), dim3(kWG), 0, s, j);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeJob& j, hipStream_t s) {
  if (j.n_vec <= 0) return hipSuccess;
  if (j.n_vec > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  const bool rot = j.signs != nullptr;
  if (j.d == 128) return rot ? decode_bits<128, true>(j, s) : decode_bits<128, false>(j, s);
  return rot ? decode_bits<64, true>(j, s) : decode_bits<64, false>(j, s);
}

}  // namespace hsq
