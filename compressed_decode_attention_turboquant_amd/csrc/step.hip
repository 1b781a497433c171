// HSQ decode step for gfx950: router + top-beta + union-set attention.
//
// [Tamarin (HSQ) summary, section 2, "Decode process": (1) a per-head router
// scores the L2 summary keys against the query; (2) the top-beta groups are
// fetched from L3 and dequantised; (3) attention runs over L1 tokens, the
// summaries and the fetched originals, with the fetched groups' summaries
// masked so nothing is counted twice.]
//
// Rotated-domain evaluation.  Every tier of one (layer, kv-head) shares the
// rotation R = H D / sqrt(d), so for a stored vector x_hat = r R^T c[code]:
//     q . x_hat = r * (R q) . c[code]
//     sum_e p_e x_hat_e = R^T sum_e p_e r_e c[code_e]
// The query is rotated once per unit (K rotation) and the attention output
// once per head (inverse V rotation); tokens are never rotated.  This is exact
// in real arithmetic; the oracle dequantises every token literally.
//
// Two kernels per step, one work-group per unit (sequence, kv-head); no
// cross-work-group communication inside a kernel (the kernel boundary orders
// the hand-over), so no device-scope fences or atomics:
//   summary_kernel  (1) streams the 3-bit summary keys: 16 summaries per MFMA
//                   tile, codes turned into fp16 pairs through a lane-replicated
//                   LDS table, split hi + lo so q_hi k_hi + q_hi k_lo + q_lo k_hi
//                   (three v_mfma_f32_16x16x32_f16) gives fp32-accurate scores;
//                   the per-head logits stay in LDS.  (2) router score per group
//                   (max or mean over the G heads), top-beta by radix select in
//                   LDS, selection written out.  (3) streams the values of the
//                   UNFETCHED summaries only (fetched rows cost no traffic),
//                   online softmax, PV on MFMA; one partial per unit.
//   token_kernel    16 tokens per tile from L1 and from the fetched L3 records;
//                   4-bit codes through a byte -> fp16-pair table (one LDS copy
//                   per lane, address built by one v_perm); QK and PV on MFMA;
//                   merge with the summary partial (log-sum-exp); inverse V
//                   rotation; output.
// Loads go through buffer descriptors scoped to the unit, so rows past the end
// and masked rows read as zero without touching memory, and the tile loops
// need no per-lane branches.  Each wave keeps the next tile's loads in flight
// while it computes the current one.
//
// Value product layout.  O^T[dims][heads] = V^T P^T would need each lane to
// hold one dimension of several tokens, but codes are stored token-major.
// Instead the MFMA rows are dimension PAIRS and k runs over (token, e):
//     A[pair r][(n, e)] = V[n][2r + e],  B[(n, e)][(h, e')] = P[h][n] [e == e']
// so C[r][(h, e')] = O[h][2r + e'].  A lane then needs, per token, a byte (two
// 4-bit codes = two dims) straight from the token's code row, and B's columns
// (h, e') are exactly the QK output columns when each head's query is placed
// in two columns (2h, 2h+1).  G <= 8 heads fill the 16 columns.
#include <cmath>

#include "hsq_device.h"
#include "hsq_internal.h"

namespace hsq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kWaves = 8;                // waves per work-group (both kernels)
constexpr int kThreads = kWaves * 64;
constexpr int kMaxG = 8;
constexpr int kNC3 = 32;                 // 3-bit table copies (lanes l, l+32 share)
constexpr int kNC4 = 64;                 // 4-bit table copies (one per lane)
constexpr int kMaxGroups = 16384;
constexpr int kMaxLogits = 12288;        // G * n_groups kept in LDS
constexpr uint32_t kFar = 0x80000000u;   // buffer offset that reads as zero
constexpr float kNegInf = -INFINITY;
constexpr float kPosInf = INFINITY;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 ld64(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x3 ld96(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ f32x4 ldf4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, ld128(r, off));
}
// four consecutive floats, each range-checked separately
__device__ __forceinline__ f32x4 ldf1x4(rsrc_t r, uint32_t off) {
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(ld32(r, off + 4 * i));
  return v;
}

__device__ __forceinline__ uint32_t h2u(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
__device__ __forceinline__ half8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(half8, u);
}
__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Runs use(i, buf) for i in [0, iters) with each buffer's loads issued two
// iterations before its use, so every wave keeps two tiles in flight.  load(i)
// is also called for i >= iters; it must then read out of bounds (buffer loads
// past num_records return zero without memory traffic).  iters is wave-uniform.
template <typename Buf, typename LoadF, typename UseF>
__device__ __forceinline__ void pipeline3(int iters, LoadF load, UseF use) {
  Buf b0, b1, b2;
  load(0, b0);
  load(1, b1);
  // whole triples only: a loop body with no exit in the middle keeps the same
  // number of loads in flight on every back edge, so the waits stay partial
  int i = 0;
  // the scheduling barriers keep the compiler from sinking the loads below
  // the previous tile's arithmetic
  for (; i + 3 <= iters; i += 3) {
    load(i + 2, b2);
    __builtin_amdgcn_sched_barrier(0);
    use(i, b0);
    load(i + 3, b0);
    __builtin_amdgcn_sched_barrier(0);
    use(i + 1, b1);
    load(i + 4, b1);
    __builtin_amdgcn_sched_barrier(0);
    use(i + 2, b2);
  }
  if (i < iters) use(i, b0);
  if (i + 1 < iters) use(i + 1, b1);
}

// Wave index as a scalar (wave-uniform for the compiler).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
__device__ __forceinline__ int wave_iters(int n_tiles, int wave) {
  return wave < n_tiles ? (n_tiles - wave + kWaves - 1) / kWaves : 0;
}

// ---------------------------------------------------------------- tables ---

// 4-bit: byte b (codes b & 15, b >> 4) -> fp16 pair; copy l at dword b*64 + l,
// so lane l's address is (b << 8) | (l << 2): one v_perm from the code dword.
__device__ void build_lut4(uint32_t* lut, const float* cb, int tid) {
  for (int i = tid; i < 256 * kNC4; i += kThreads) {
    const int e = i / kNC4;
    lut[i] = h2u((_Float16)cb[e & 15], (_Float16)cb[e >> 4]);
  }
}
// byte K of w as a table address for this lane
template <int K>
__device__ __forceinline__ uint32_t lut4_addr(uint32_t w, uint32_t lane4) {
  // bytes of {lane4 (sel 4..7), w (sel 0..3)}: result = [lane4.b0, w.bK, 0, 0]
  return __builtin_amdgcn_perm(lane4, w, 0x0c0c0004u | (uint32_t(K) << 8));
}
__device__ __forceinline__ uint32_t lut4_rd(const uint32_t* lut, uint32_t addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + addr);
}

// 3-bit: 6-bit field e (codes e & 7, e >> 3) -> hi fp16 pair at lut[e*32 + l%32]
// and lo fp16 pair 64*32 dwords further (same address + 8 KB), c = hi + lo to
// ~2^-22 relative.
__device__ void build_lut3(uint32_t* lut, const float* cb, int tid) {
  for (int i = tid; i < 64 * kNC3; i += kThreads) {
    const int e = i / kNC3;
    const float c0 = cb[e & 7], c1 = cb[e >> 3];
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
    lut[i] = h2u(h0, h1);
    lut[64 * kNC3 + i] = h2u(l0, l1);
  }
}
__device__ __forceinline__ uint32_t lut3_addr(uint32_t e, uint32_t lane4) {
  return (e << 7) | lane4;  // lane4 = (lane & 31) << 2
}
__device__ __forceinline__ uint32_t lut3_hi(const uint32_t* lut, uint32_t addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + addr);
}
__device__ __forceinline__ uint32_t lut3_lo(const uint32_t* lut, uint32_t addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + addr +
                                            64 * kNC3 * 4);
}

// -------------------------------------------------------- query rotation ---

// qf[h][i] = mult * (H D q_h)[i] for h < G, 0 for G <= h < 8, on the first
// 8*D/8 threads (whole waves).
template <int D>
__device__ void rotate_queries(const float* q, const uint32_t* mask, int G, float mult, float* qf,
                               int tid) {
  constexpr int LPV = D / 8;
  if (tid < kMaxG * LPV) {
    const int h = tid / LPV, sub = tid % LPV;
    float v[8];
    if (h < G) {
      const float4* p = reinterpret_cast<const float4*>(q + h * D + 8 * sub);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      const uint32_t sb = sign_byte(mask, sub);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = flip(v[k], (sb >> k) & 1u);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = 0.f;
    }
    fwht8xlanes<LPV>(v, sub);
#pragma unroll
    for (int k = 0; k < 8; ++k) qf[h * D + 8 * sub + k] = v[k] * mult;
  }
}

// B operand of the QK products: lane (c, gq) holds head c/2, dims
// gq*D/4 + 8m + j for k-chunk m; hi/lo fp16 split of the fp32 rotated query.
template <int D>
__device__ void query_operands(const float* qf, int lane, half8 (&hi)[D / 32],
                               half8 (&lo)[D / 32]) {
  const int c = lane & 15, gq = lane >> 4, h = c >> 1;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qf[h * D + gq * (D / 4) + 8 * m + j];
      const _Float16 xh = (_Float16)x;
      hi[m][j] = xh;
      lo[m][j] = (_Float16)(x - (float)xh);
    }
  }
}

// ---------------------------------------------------------- online softmax ---

template <int D>
struct Online {
  float m;   // running max of this lane's column (equal on the 4 row groups)
  float l;   // this lane's share of the denominator (its 4 rows)
  f32x4 O[D / 32];
  __device__ void init() {
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Fold in 4 logits of this lane (rows 4gq+i); p = exp(lg - m_new).
  __device__ __forceinline__ void update(const float (&lg)[4], float (&p)[4]) {
    float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    // rescale only when some column's running max moved (wave-uniform branch)
    if (__builtin_amdgcn_ballot_w64(mn > m)) {
      const float alpha = (mn > m) ? __expf(m - ms) : 1.f;
      l *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) O[t] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __expf(lg[i] - ms);
    m = mn;
  }
};

// PV with 4-bit values: va[j] = this lane's value bits of token 4gq+j, p[j] =
// weight (times the value norm) of token 4gq+j for this lane's column (h, e').
template <int D>
__device__ __forceinline__ void pv4(const uint32_t (&va)[4], const float (&p)[4], int lane,
                                    uint32_t lane4, const uint32_t* lut4, f32x4 (&O)[D / 32]) {
  const uint32_t sh = (lane & 1) ? 16u : 0u;
  uint32_t pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p[j]) << sh;
  const half8 b = as_h8(pb[0], pb[1], pb[2], pb[3]);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    uint32_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t addr;
      if (t == 0) addr = lut4_addr<0>(va[j], lane4);
      else if (t == 1) addr = lut4_addr<1>(va[j], lane4);
      else if (t == 2) addr = lut4_addr<2>(va[j], lane4);
      else addr = lut4_addr<3>(va[j], lane4);
      a[j] = lut4_rd(lut4, addr);
    }
    O[t] = mfma16(as_h8(a[0], a[1], a[2], a[3]), b, O[t]);
  }
}

// PV with 3-bit values (hi part of the table; V needs no split).
template <int D>
__device__ __forceinline__ void pv3(const uint32_t (&va)[4], const float (&p)[4], int lane,
                                    uint32_t lane4, const uint32_t* lut3, f32x4 (&O)[D / 32]) {
  const uint32_t sh = (lane & 1) ? 16u : 0u;
  uint32_t pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p[j]) << sh;
  const half8 b = as_h8(pb[0], pb[1], pb[2], pb[3]);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    uint32_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = lut3_hi(lut3, lut3_addr((va[j] >> (6 * t)) & 63u, lane4));
    O[t] = mfma16(as_h8(a[0], a[1], a[2], a[3]), b, O[t]);
  }
}

// Combine the waves' states; result per head written to dst[h][D+2] as
// [m, l, O[0..D)] (dst may be LDS or global).  scratch: kWaves*kMaxG*(D+2) floats.
template <int D>
__device__ void combine_waves(const Online<D>& st, int G, float* scratch, float* dst, int tid) {
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, gq = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  constexpr int T = D / 32;
  const int h = c >> 1;
  float* w = scratch + (wave * kMaxG + h) * (D + 2);
  if (h < G) {
    if (gq == 0 && !(c & 1)) {
      w[0] = st.m;
      w[1] = l;
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[2 + 2 * (T * (4 * gq + i) + t) + (c & 1)] = st.O[t][i];
  }
  __syncthreads();
  for (int k = tid; k < G * (D + 2); k += kThreads) {
    const int hh = k / (D + 2), e = k % (D + 2);
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, scratch[(v * kMaxG + hh) * (D + 2)]);
    float acc = 0.f;
    if (e > 0) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float* s = scratch + (v * kMaxG + hh) * (D + 2);
        const float wgt = (s[0] == kNegInf) ? 0.f : __expf(s[0] - M);
        acc += wgt * s[e];
      }
    }
    dst[k] = (e == 0) ? M : acc;
  }
  __syncthreads();
}

// ------------------------------------------------------------ top-beta ------

// Ordered uint32 key of a float: larger float <-> larger key.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the work-group.
__device__ int block_exclusive_scan(int v, int* tmp, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  __syncthreads();
  return base + x - v;
}

// Top-beta of keys[0..ng): sel[0..beta) ascending group ids.  Radix select (4
// passes of 8 bits, most significant first) finds the key of the beta-th
// largest score and how many of its ties to take; an in-order scan then emits
// the selected ids, ties resolved to the lower index.  0 < beta < ng.
__device__ void top_beta(const uint32_t* keys, int ng, int beta, int* hist, int* tmp,
                         int32_t* sel, int tid) {
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_need;
  if (tid == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_need = beta;
  }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kThreads) hist[b] = 0;
    __syncthreads();
    const uint32_t pre = s_prefix, msk = s_mask;
    for (int g = tid; g < ng; g += kThreads) {
      const uint32_t k = keys[g];
      if ((k & msk) == pre) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending order)
      int cnt[4], sum = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cnt[k] = hist[255 - 4 * tid - k];
        sum += cnt[k];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (tid >= o) incl += y;
      }
      const int need = s_need;
      const int excl = incl - sum;
      if (excl < need && incl >= need) {
        int acc = excl;
        for (int k = 0; k < 4; ++k) {
          if (acc + cnt[k] >= need) {
            const uint32_t bin = 255u - 4u * tid - k;
            s_prefix = pre | (bin << shift);
            s_mask = msk | (255u << shift);
            s_need = need - acc;
            break;
          }
          acc += cnt[k];
        }
      }
    }
    __syncthreads();
  }
  const uint32_t kth = s_prefix;
  const int ties_needed = s_need;  // keys equal to kth to take
  const int per = (ng + kThreads - 1) / kThreads;
  const int lo = min(tid * per, ng), hi = min(lo + per, ng);
  int n_eq = 0;
  for (int g = lo; g < hi; ++g) n_eq += keys[g] == kth;
  const int eq_base = block_exclusive_scan(n_eq, tmp, tid);
  int n_sel = 0, e = eq_base;
  for (int g = lo; g < hi; ++g) {
    const uint32_t k = keys[g];
    if (k > kth) ++n_sel;
    else if (k == kth) n_sel += (e++ < ties_needed);
  }
  int pos = block_exclusive_scan(n_sel, tmp, tid);
  e = eq_base;
  for (int g = lo; g < hi; ++g) {
    const uint32_t k = keys[g];
    bool take = k > kth;
    if (k == kth) take = (e++ < ties_needed);
    if (take) sel[pos++] = g;
  }
  __syncthreads();
}

// Inverse of fkey.
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Bucket of a score in 256 equal steps of [lo, hi]: a non-decreasing map of
// the score, so a larger key never lands in a lower bucket.
__device__ __forceinline__ int score_bucket(uint32_t key, float lo, float scale) {
  const float b = (key_float(key) - lo) * scale;
  return (int)fminf(fmaxf(b, 0.f), 255.f);
}

constexpr int kCandCap = 1024;  // candidates the bucket pass can rank

// Top-beta by a score histogram, 0 < beta < ng.  Every bucket above the one
// that holds the beta-th largest score is taken whole; the scores in that
// bucket are ranked exactly by (key descending, index ascending), which is
// the order of the full sort.  Sets the selected groups' bits in fmask (zero
// on entry) and returns true, or returns false with fmask untouched when the
// threshold bucket holds more than kCandCap scores.
__device__ bool select_top_hist(const uint32_t* keys, int ng, int beta, float lo, float hi,
                                int* hist, uint2* cand, uint32_t* fmask, int* st, int tid) {
  const float scale = (hi > lo) ? 256.f / (hi - lo) : 0.f;
  for (int g = tid; g < ng; g += kThreads) atomicAdd(&hist[score_bucket(keys[g], lo, scale)], 1);
  __syncthreads();
  if (tid < 64) {  // lane l owns buckets 255-4l .. 252-4l (descending)
    int cnt[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cnt[k] = hist[255 - 4 * tid - k];
      sum += cnt[k];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (tid >= o) incl += y;
    }
    const int excl = incl - sum;
    if (excl < beta && incl >= beta) {
      int acc = excl;
      for (int k = 0; k < 4; ++k) {
        if (acc + cnt[k] >= beta) {
          st[0] = 255 - 4 * tid - k;  // threshold bucket
          st[1] = beta - acc;         // how many of its scores to take
          break;
        }
        acc += cnt[k];
      }
    }
  }
  __syncthreads();
  const int bt = st[0], need = st[1];
  if (hist[bt] > kCandCap) return false;  // uniform: every thread reads the same count
  for (int g = tid; g < ng; g += kThreads) {
    const uint32_t k = keys[g];
    const int b = score_bucket(k, lo, scale);
    if (b > bt) atomicOr(&fmask[g >> 5], 1u << (g & 31));
    else if (b == bt) cand[atomicAdd(&st[2], 1)] = make_uint2((uint32_t)g, k);
  }
  __syncthreads();
  const int nc = st[2];
  for (int i = tid; i < nc; i += kThreads) {
    const uint2 me = cand[i];
    int rank = 0;
    for (int j = 0; j < nc; ++j) {
      const uint2 o = cand[j];
      rank += (o.y > me.y) || (o.y == me.y && o.x < me.x);
    }
    if (rank < need) atomicOr(&fmask[me.x >> 5], 1u << (me.x & 31));
  }
  __syncthreads();
  return true;
}

// Writes the set bits of fmask (the selection) as ascending group ids to
// idx[0 .. count); run by one wave.
__device__ void emit_selection(const uint32_t* fmask, int words, int32_t* idx, int lane) {
  const int per = (words + 63) / 64;
  const int w0 = min(lane * per, words), w1 = min(w0 + per, words);
  int n = 0;
  for (int w = w0; w < w1; ++w) n += __popc(fmask[w]);
  int incl = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  int pos = incl - n;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = fmask[w];
    while (m) {
      const int b = __ffs(m) - 1;
      idx[pos++] = 32 * w + b;
      m &= m - 1u;
    }
  }
}

// -------------------------------------------------------- summary kernel ---

struct SumArgs {
  const float* q;
  const uint8_t* l2k; const float* l2k_n; const uint8_t* l2v; const float* l2v_n;
  const uint32_t* k_signs; const float* cb3;
  float scale, bias;
  int agg, Hkv, G, ng, beta;
  int want_topk;           // route: compute scores + top-beta
  int want_partial;        // attention: summary partial
  const int32_t* given;    // fetched set to mask when not selecting here, or null
  float* scores_out;       // optional [units][ng]
  int32_t* idx;            // [units][beta] selection out (want_topk)
  float* part;             // [units][G][D+2] summary partial out
};

// 6-bit field at a compile-time bit position of a small word array.
template <int BIT>
__device__ __forceinline__ uint32_t field6(const uint32_t* w) {
  constexpr int k = BIT >> 5, s = BIT & 31;
  if constexpr (s <= 26) {
    return (w[k] >> s) & 63u;
  } else {
    return __builtin_amdgcn_alignbit(w[k + 1], w[k], s) & 63u;
  }
}

template <int D, int P>
__device__ __forceinline__ void key3_pairs(const uint32_t* kw, const uint32_t* lut, uint32_t lane4,
                                           uint32_t (&hi)[D / 8], uint32_t (&lo)[D / 8]) {
  if constexpr (P < D / 8) {
    const uint32_t a = lut3_addr(field6<6 * P>(kw), lane4);
    hi[P] = lut3_hi(lut, a);
    lo[P] = lut3_lo(lut, a);
    key3_pairs<D, P + 1>(kw, lut, lane4, hi, lo);
  }
}

// QK of 16 summaries: three-term split product.  kw: this lane's 3D/4 key bits
// (summary lane&15, dims gq*D/4 ..) from bit 0.
template <int D>
__device__ __forceinline__ f32x4 qk3(const uint32_t (&kw)[4], const half8 (&qh)[D / 32],
                                     const half8 (&ql)[D / 32], const uint32_t* lut,
                                     uint32_t lane4) {
  uint32_t hi[D / 8], lo[D / 8];
  key3_pairs<D, 0>(kw, lut, lane4, hi, lo);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const half8 ah = as_h8(hi[4 * m], hi[4 * m + 1], hi[4 * m + 2], hi[4 * m + 3]);
    const half8 al = as_h8(lo[4 * m], lo[4 * m + 1], lo[4 * m + 2], lo[4 * m + 3]);
    acc = mfma16(ah, qh[m], acc);
    acc = mfma16(ah, ql[m], acc);
    acc = mfma16(al, qh[m], acc);
  }
  return acc;
}

// Keys of tile t (16 summaries): this lane's key bits and the key norms of rows
// 4gq .. 4gq+3.
struct KeyTile {
  uint32_t kw[4];
  f32x4 kn;
};
template <int D>
__device__ __forceinline__ void load_keys(rsrc_t rk, rsrc_t rn, int t, int lane, KeyTile& T) {
  constexpr int CB3 = 3 * D / 8;
  const int n = lane & 15, gq = lane >> 4;
  const uint32_t row = (uint32_t)(16 * t + n) * CB3;
  if constexpr (D == 128) {  // 96 bits at byte 12*gq
    const u32x3 w = ld96(rk, row + 12 * gq);
    T.kw[0] = w.x; T.kw[1] = w.y; T.kw[2] = w.z; T.kw[3] = 0u;
  } else {                   // 48 bits at bit 48*gq: raw dwords, aligned by key_bits
    const u32x2 w = ld64(rk, row + 4 * ((3 * gq) >> 1));
    T.kw[0] = w.x; T.kw[1] = w.y; T.kw[2] = 0u; T.kw[3] = 0u;
  }
  T.kn = ldf1x4(rn, (uint32_t)(16 * t + 4 * gq) * 4);
}

// This lane's key bits from the words load_keys left (the loads stay free of
// arithmetic so that no wait is forced before the tile is used).
template <int D>
__device__ __forceinline__ void key_bits(const uint32_t (&w)[4], int lane, uint32_t (&kw)[4]) {
  if constexpr (D == 128) {
    kw[0] = w[0]; kw[1] = w[1]; kw[2] = w[2]; kw[3] = 0u;
  } else {
    const uint32_t s = ((lane >> 4) & 1) ? 16u : 0u;
    kw[0] = __builtin_amdgcn_alignbit(w[1], w[0], s);
    kw[1] = w[1] >> s;
    kw[2] = 0u; kw[3] = 0u;
  }
}

// Values of tile t: the dword of row 4gq+j that holds this lane's value bits
// (dims [2T*rho, 2T*rho + 2T), T = D/32; shifted into place by the consumer)
// and the rows' norms; rows flagged in `skip` read as zero.
struct ValTile {
  uint32_t va[4];
  f32x4 vn;
  uint32_t skip;
};
// The dword holding this lane's value bits starts at byte min(bit/8, RB-4)
// (so it never crosses the end of the row; buffer loads need only byte
// alignment); val_shift is where the bits start in it.
template <int D>
__device__ __forceinline__ uint32_t val_byte(int lane) {
  constexpr int RB = 3 * D / 8;        // bytes per row
  constexpr int BITS = 6 * (D / 32);   // bits per lane per row
  return (uint32_t)min((BITS * (lane & 15)) >> 3, RB - 4);
}
template <int D>
__device__ __forceinline__ uint32_t val_shift(int lane) {
  constexpr int BITS = 6 * (D / 32);
  return (uint32_t)(BITS * (lane & 15)) - 8u * val_byte<D>(lane);
}
template <int D>
__device__ __forceinline__ void load_vals(rsrc_t rv, rsrc_t rvn, int t, int lane, uint32_t skip,
                                          ValTile& T) {
  constexpr int RB = 3 * D / 8;
  const int gq = lane >> 4;
  const uint32_t wofs = val_byte<D>(lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t row = (uint32_t)(16 * t + 4 * gq + j) * RB;
    T.va[j] = ld32(rv, ((skip >> j) & 1u) ? kFar : row + wofs);
  }
  T.vn = ldf1x4(rvn, (uint32_t)(16 * t + 4 * gq) * 4);
}

template <int D>
__global__ __launch_bounds__(kThreads) void summary_kernel(SumArgs a) {
  constexpr int CB3 = 3 * D / 8;
  extern __shared__ __align__(16) char smem[];
  __shared__ float s_cb[8];
  __shared__ int s_tmp[kWaves];
  __shared__ int s_sel[4];
  __shared__ float s_lo[kWaves], s_hi[kWaves];
  // layout: [lut3 16 KB][qf 8*D f32][logits G*ngp f32][keys ngp u32][hist 256]
  //         [fetched bitmap][dummy 64x4 f32][selection scratch: candidates
  //         (uint2) or, in the fallback, the selected ids]; the wave-combine
  //         scratch reuses the front once the tiles are done.
  const int ngp = (a.ng + 15) & ~15;
  uint32_t* lut3 = reinterpret_cast<uint32_t*>(smem);
  float* qf = reinterpret_cast<float*>(smem + 64 * kNC3 * 8);
  float* logits = qf + kMaxG * D;
  uint32_t* keys = reinterpret_cast<uint32_t*>(logits + a.G * ngp);
  int* hist = reinterpret_cast<int*>(keys + ngp);
  uint32_t* fmask = reinterpret_cast<uint32_t*>(hist + 256);
  float* dummy = reinterpret_cast<float*>(fmask + (((ngp + 31) / 32 + 3) & ~3));  // [64][4]
  uint2* cand = reinterpret_cast<uint2*>(dummy + 256);
  int32_t* sel = reinterpret_cast<int32_t*>(cand);
  float* scratch = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int unit = blockIdx.x;
  const int kvh = unit % a.Hkv;
  const uint32_t lane4 = (uint32_t)(lane & 31) << 2;
  const int c = lane & 15, gq = lane >> 4;

  const rsrc_t rk = make_rsrc(a.l2k + (size_t)unit * a.ng * CB3, (uint32_t)a.ng * CB3);
  const rsrc_t rkn = make_rsrc(a.l2k_n + (size_t)unit * a.ng, (uint32_t)a.ng * 4);

  if (tid < 8) s_cb[tid] = a.cb3[tid];
  rotate_queries<D>(a.q + (size_t)unit * a.G * D, a.k_signs + kvh * (D / 32), a.G,
                    a.scale * rsqrtf((float)D), qf, tid);
  const int words = (ngp + 31) >> 5;
  for (int w = tid; w < words; w += kThreads) fmask[w] = 0u;
  for (int b = tid; b < 256; b += kThreads) hist[b] = 0;
  if (tid < 4) s_sel[tid] = 0;
  __syncthreads();
  build_lut3(lut3, s_cb, tid);
  half8 qh[D / 32], ql[D / 32];
  query_operands<D>(qf, lane, qh, ql);
  __syncthreads();

  // (1) keys -> per-head logits in LDS (column 2h holds head h)
  const int n_tiles = ngp >> 4;
  // lanes that hold no head's logits store into a dummy slot (no branch)
  const bool writer = !(c & 1) && (c >> 1) < a.G;
  float* lw = writer ? logits + (c >> 1) * ngp + 4 * gq : dummy + 4 * lane;
  {
    pipeline3<KeyTile>(
        wave_iters(n_tiles, wave),
        [&](int i, KeyTile& T) { load_keys<D>(rk, rkn, wave + i * kWaves, lane, T); },
        [&](int i, const KeyTile& T) {
          uint32_t kw[4];
          key_bits<D>(T.kw, lane, kw);
          const f32x4 acc = qk3<D>(kw, qh, ql, lut3, lane4);
          *reinterpret_cast<f32x4*>(lw + (writer ? 16 * (wave + i * kWaves) : 0)) = acc * T.kn;
        });
  }
  __syncthreads();

  // (2) router scores, top-beta, fetched bitmap
  if (a.want_topk) {
    const float inv_g = 1.f / (float)a.G;
    float lo = kPosInf, hi = kNegInf;
    for (int g = tid; g < a.ng; g += kThreads) {
      float v = logits[g];
      if (a.agg == HSQ_AGG_MAX) {
        for (int h = 1; h < a.G; ++h) v = fmaxf(v, logits[h * ngp + g]);
      } else {
        for (int h = 1; h < a.G; ++h) v += logits[h * ngp + g];
        v *= inv_g;
      }
      keys[g] = fkey(v);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
      if (a.scores_out) a.scores_out[(size_t)unit * a.ng + g] = v;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o, 64));
      hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    if (lane == 0) {
      s_lo[wave] = lo;
      s_hi[wave] = hi;
    }
    __syncthreads();
    for (int w = 0; w < kWaves; ++w) {
      lo = fminf(lo, s_lo[w]);
      hi = fmaxf(hi, s_hi[w]);
    }
    if (a.beta >= a.ng) {
      for (int w = tid; w < words; w += kThreads) {
        const int left = a.ng - 32 * w;
        fmask[w] = left >= 32 ? 0xffffffffu : (left <= 0 ? 0u : ((1u << left) - 1u));
      }
    } else if (a.beta > 0) {
      if (!select_top_hist(keys, a.ng, a.beta, lo, hi, hist, cand, fmask, s_sel, tid)) {
        top_beta(keys, a.ng, a.beta, hist, s_tmp, sel, tid);
        for (int i = tid; i < a.beta; i += kThreads) atomicOr(&fmask[sel[i] >> 5], 1u << (sel[i] & 31));
      }
    }
    __syncthreads();
    if (wave == 0) emit_selection(fmask, words, a.idx + (size_t)unit * a.beta, lane);
  } else if (a.given) {
    for (int i = tid; i < a.beta; i += kThreads) {
      const int g = a.given[(size_t)unit * a.beta + i];
      if (g >= 0 && g < a.ng) atomicOr(&fmask[g >> 5], 1u << (g & 31));
    }
  }
  __syncthreads();
  if (!a.want_partial) return;

  // (3) values of the unfetched summaries -> partial
  const rsrc_t rv = make_rsrc(a.l2v + (size_t)unit * a.ng * CB3, (uint32_t)a.ng * CB3);
  const rsrc_t rvn = make_rsrc(a.l2v_n + (size_t)unit * a.ng, (uint32_t)a.ng * 4);
  Online<D> st;
  st.init();
  const float* lrow = logits + min(c >> 1, a.G - 1) * ngp + 4 * gq;
  auto skip_of = [&](int t) -> uint32_t {  // rows 4gq+j of tile t fetched or past the end
    const int g0 = 16 * max(min(t, n_tiles - 1), 0) + 4 * gq;
    const uint32_t fm = (fmask[g0 >> 5] >> (g0 & 31)) & 15u;  // g0 % 4 == 0: one word
    if (t >= n_tiles) return 15u;
    const int valid = a.ng - g0;
    const uint32_t vm = valid >= 4 ? 15u : (valid <= 0 ? 0u : ((1u << valid) - 1u));
    return fm | (~vm & 15u);
  };
  const uint32_t vsh = val_shift<D>(lane);
  auto consume = [&](int t, const ValTile& V, uint32_t skip) {
    const f32x4 lg4 = *reinterpret_cast<const f32x4*>(lrow + 16 * t);
    float lg[4], p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = ((skip >> i) & 1u) ? kNegInf : lg4[i] + a.bias;
    st.update(lg, p);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      psum += p[i];
      p[i] *= V.vn[i];
    }
    st.l += psum;
    uint32_t va[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) va[j] = V.va[j] >> vsh;
    pv3<D>(va, p, lane, lane4, lut3, st.O);
  };
  {
    pipeline3<ValTile>(
        wave_iters(n_tiles, wave),
        [&](int i, ValTile& V) {
          const int t = wave + i * kWaves;
          V.skip = skip_of(t);
          load_vals<D>(rv, rvn, t, lane, V.skip, V);
        },
        [&](int i, const ValTile& V) { consume(wave + i * kWaves, V, V.skip); });
  }
  __syncthreads();  // the tables and logits are no longer needed: reuse as scratch
  combine_waves<D>(st, a.G, scratch, a.part + (size_t)unit * a.G * (D + 2), tid);
}

// ----------------------------------------------------------- token kernel ---

struct TokArgs {
  const float* q;
  const uint8_t* l1k; const float* l1k_n; const uint8_t* l1v; const float* l1v_n;
  const uint8_t* l3; int l3_staged;
  const int32_t* idx;
  const uint32_t* k_signs; const uint32_t* v_signs; const float* cb4;
  float scale;
  int Hkv, G, n1, ng, group_n, beta;
  const float* part;       // summary partial per unit, or null when there are none
  float* out;
};

struct TokTile {
  u32x4 kw;        // key code dwords of token row lane&15 (D=64 uses .x, .y)
  f32x4 kn;        // key norms of rows 4gq+i
  f32x4 vn;        // value norms of rows 4gq+i
  uint32_t va[4];  // value bits of rows 4gq+j for lane rho = lane&15
  uint32_t ok;     // bit i: row 4gq+i is a real token
};

struct TokRsrc {
  rsrc_t l1k, l1kn, l1v, l1vn, l3;
};

// Tile t: L1 rows 16t .. 16t+15 for t < n1t, else the fetched archive groups
// of tile t - n1t (N = 16: one group; N = 8: two).  Both kinds issue the same
// loads in the same order; only the buffers (picked by the wave-uniform test)
// and the per-lane offsets differ, so the loads sit in straight-line code.
template <int D>
__device__ __forceinline__ void load_tok(const TokArgs& a, const TokRsrc& R, const int32_t* sel,
                                         int t, int n1t, int lane, TokTile& T) {
  constexpr int CB = D / 2;
  constexpr uint32_t KB = D / 8;  // key code bytes per lane
  const int n = lane & 15, gq = lane >> 4;
  const bool l1 = t < n1t;
  // archive record = [K codes N*CB][K norms N*4][V codes N*CB][V norms N*4]
  const int N = a.group_n;
  const uint32_t rec = (uint32_t)N * (D + 8);
  const int f = t - n1t;
  auto rec_off = [&](int slot) -> uint32_t {
    const int g = a.l3_staged ? slot : sel[min(max(slot, 0), max(a.beta - 1, 0))];
    const int lim = a.l3_staged ? a.beta : a.ng;
    return (slot >= 0 && slot < a.beta && g >= 0 && g < lim) ? (uint32_t)g * rec : kFar;
  };
  // key row n: slot and token within the group; rows 4gq .. 4gq+3 lie in one
  // group (N is a multiple of 4)
  const int sk = (N == 16) ? f : 2 * f + (n >> 3);
  const int tk = (N == 16) ? n : (n & 7);
  const int sr = (N == 16) ? f : 2 * f + (gq >> 1);
  const int tr = (N == 16) ? 4 * gq : 4 * (gq & 1);
  const uint32_t bk = rec_off(sk), br = rec_off(sr);
  const bool okr = br != kFar;
  const uint32_t r0 = (uint32_t)(16 * t);
  // an offset built on kFar stays past the end of every buffer (reads zero)
  const uint32_t ko = l1 ? (r0 + n) * CB + KB * gq : bk + tk * CB + KB * gq;
  const uint32_t kno = l1 ? (r0 + 4 * gq) * 4 : br + N * CB + 4 * tr;
  const uint32_t vno = l1 ? (r0 + 4 * gq) * 4 : br + N * (2 * CB + 4) + 4 * tr;
  const uint32_t vo = (l1 ? (r0 + 4 * gq) * CB : br + N * (CB + 4) + tr * CB) +
                      ((D == 128) ? 4 * n : 4 * (n >> 1));
  const rsrc_t rk = l1 ? R.l1k : R.l3, rkn = l1 ? R.l1kn : R.l3;
  const rsrc_t rv = l1 ? R.l1v : R.l3, rvn = l1 ? R.l1vn : R.l3;
  if constexpr (D == 128) {
    T.kw = ld128(rk, ko);
  } else {
    const u32x2 w = ld64(rk, ko);
    T.kw = u32x4{w.x, w.y, 0u, 0u};
  }
  T.kn = ldf1x4(rkn, kno);
  T.vn = ldf1x4(rvn, vno);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    T.va[j] = ld32(rv, vo + j * CB);  // D = 64: consume_tok takes the lane's half
  }
  const int valid = a.n1 - (int)(r0 + 4 * gq);
  const uint32_t ok1 = valid >= 4 ? 15u : (valid <= 0 ? 0u : ((1u << valid) - 1u));
  T.ok = l1 ? ok1 : (okr ? 15u : 0u);
}

template <int D>
__device__ __forceinline__ void consume_tok(const TokTile& T, const half8 (&qh)[D / 32],
                                            const uint32_t* lut4, int lane, uint32_t lane4,
                                            Online<D>& st) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const uint32_t w = T.kw[m];
    const half8 av = as_h8(lut4_rd(lut4, lut4_addr<0>(w, lane4)),
                           lut4_rd(lut4, lut4_addr<1>(w, lane4)),
                           lut4_rd(lut4, lut4_addr<2>(w, lane4)),
                           lut4_rd(lut4, lut4_addr<3>(w, lane4)));
    acc = mfma16(av, qh[m], acc);
  }
  float lg[4], p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lg[i] = ((T.ok >> i) & 1u) ? acc[i] * T.kn[i] : kNegInf;
  st.update(lg, p);
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    psum += p[i];
    p[i] *= T.vn[i];
  }
  st.l += psum;
  uint32_t va[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) va[j] = (D == 128) ? T.va[j] : (T.va[j] >> (16 * (lane & 1)));
  pv4<D>(va, p, lane, lane4, lut4, st.O);
}

// at most 128 VGPRs so that two work-groups (the LDS limit) fit on a CU
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void token_kernel(TokArgs a) {
  constexpr int CB = D / 2;
  extern __shared__ __align__(16) char smem[];
  __shared__ float s_cb[16];
  // layout: [lut4 64 KB][qf 8*D f32][sel beta]; the combine scratch reuses the
  // front once the tiles are done.
  uint32_t* lut4 = reinterpret_cast<uint32_t*>(smem);
  float* qf = reinterpret_cast<float*>(smem + 256 * kNC4 * 4);
  int32_t* sel = reinterpret_cast<int32_t*>(qf + kMaxG * D);
  float* scratch = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int unit = blockIdx.x;
  const int kvh = unit % a.Hkv;
  const uint32_t lane4 = (uint32_t)lane << 2;

  if (tid < 16) s_cb[tid] = a.cb4[tid];
  if (!a.l3_staged)
    for (int i = tid; i < a.beta; i += kThreads) sel[i] = a.idx[(size_t)unit * a.beta + i];
  rotate_queries<D>(a.q + (size_t)unit * a.G * D, a.k_signs + kvh * (D / 32), a.G,
                    a.scale * rsqrtf((float)D), qf, tid);
  __syncthreads();
  build_lut4(lut4, s_cb, tid);
  half8 qh[D / 32], ql[D / 32];
  query_operands<D>(qf, lane, qh, ql);
  __syncthreads();

  const size_t o1 = (size_t)unit * a.n1;
  const size_t rec = (size_t)a.group_n * (D + 8);
  const int recs = a.l3_staged ? a.beta : a.ng;
  const TokRsrc R{make_rsrc(a.l1k + o1 * CB, (uint32_t)a.n1 * CB),
                  make_rsrc(a.l1k_n + o1, (uint32_t)a.n1 * 4),
                  make_rsrc(a.l1v + o1 * CB, (uint32_t)a.n1 * CB),
                  make_rsrc(a.l1v_n + o1, (uint32_t)a.n1 * 4),
                  make_rsrc(a.l3 + (size_t)unit * recs * rec, (uint32_t)(recs * rec))};

  const int n1t = (a.n1 + 15) / 16;
  const int nft = (a.group_n == 16) ? a.beta : (a.beta + 1) / 2;
  const int total = n1t + nft;
  Online<D> st;
  st.init();
  {
    pipeline3<TokTile>(
        wave_iters(total, wave),
        [&](int i, TokTile& T) {
          load_tok<D>(a, R, sel, wave + i * kWaves, n1t, lane, T);
        },
        [&](int i, const TokTile& T) { consume_tok<D>(T, qh, lut4, lane, lane4, st); });
  }
  __syncthreads();  // the table is no longer needed: reuse as scratch
  float* mine = scratch + kWaves * kMaxG * (D + 2);  // [G][D+2] this unit's token partial
  combine_waves<D>(st, a.G, scratch, mine, tid);

  // merge with the summary partial, normalise
  float* o = mine + kMaxG * (D + 2);  // [G][D]
  const float* ps = a.part ? a.part + (size_t)unit * a.G * (D + 2) : nullptr;
  for (int k = tid; k < a.G * D; k += kThreads) {
    const int h = k / D, e = k % D;
    const float* pm = mine + h * (D + 2);
    const float m1 = pm[0], l1 = pm[1], v1 = pm[2 + e];
    float m2 = kNegInf, l2 = 0.f, v2 = 0.f;
    if (ps) {
      m2 = ps[h * (D + 2)];
      l2 = ps[h * (D + 2) + 1];
      v2 = ps[h * (D + 2) + 2 + e];
    }
    const float M = fmaxf(m1, m2);
    const float w1 = (m1 == kNegInf) ? 0.f : __expf(m1 - M);
    const float w2 = (m2 == kNegInf) ? 0.f : __expf(m2 - M);
    const float L = w1 * l1 + w2 * l2;
    o[k] = (L > 0.f) ? (w1 * v1 + w2 * v2) / L : 0.f;
  }
  __syncthreads();
  // inverse V rotation: out = D H o / sqrt(D)
  constexpr int LPV = D / 8;
  if (tid < kMaxG * LPV) {
    const int h = tid / LPV, sub = tid % LPV;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (h < a.G) ? o[h * D + 8 * sub + k] : 0.f;
    fwht8xlanes<LPV>(v, sub);
    if (h < a.G) {
      const uint32_t sb = sign_byte(a.v_signs + kvh * (D / 32), sub);
      const float sc = rsqrtf((float)D);
      float* dst = a.out + ((size_t)unit * a.G + h) * D + 8 * sub;
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = flip(v[k] * sc, (sb >> k) & 1u);
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t summary_smem(int D, const StepShape& s) {
  const size_t ngp = (size_t)((s.n_groups + 15) & ~15);
  const size_t body = 64 * kNC3 * 8 + (size_t)kMaxG * D * 4 + (size_t)s.G * ngp * 4 + ngp * 4 +
                      256 * 4 + (((ngp + 31) / 32 + 3) & ~size_t(3)) * 4 + 64 * 16 +
                      std::max((size_t)s.beta * 4, (size_t)std::min<size_t>(ngp, kCandCap) * 8);
  const size_t comb = (size_t)kWaves * kMaxG * (D + 2) * 4;
  return std::max(body, comb);
}

size_t token_smem(int D, const StepShape& s) {
  const size_t body = 256 * kNC4 * 4 + (size_t)kMaxG * D * 4 + (size_t)((s.beta + 4) & ~3) * 4;
  const size_t comb = (size_t)kWaves * kMaxG * (D + 2) * 4 + (size_t)kMaxG * (D + 2) * 4 +
                      (size_t)kMaxG * D * 4;
  return std::max(body, comb);
}

}  // namespace

Workspace plan_workspace(const StepShape& s) {
  Workspace w{};
  const int units = s.B * s.Hkv;
  size_t off = 0;
  w.idx_off = off;  off = align256(off + (size_t)units * std::max(s.beta, 1) * 4);
  w.part_off = off; off = align256(off + (size_t)units * s.G * (s.d + 2) * 4);
  w.total = off;
  return w;
}

int step_limits_ok(const StepShape& s) {
  const size_t rec = (size_t)s.group_n * (s.d + 8);
  return s.n_groups <= kMaxGroups && s.G * ((s.n_groups + 15) & ~15) <= kMaxLogits &&
         (size_t)s.n_groups * rec < 0x7fffffffu && (size_t)s.n_l1 * s.d < 0x7fffffffu;
}

template <int D>
hipError_t summary_d(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                     int mode, const int32_t* given, float* scores_out, int32_t* idx_out,
                     hipStream_t st) {
  SumArgs a{};
  a.q = t.q; a.l2k = t.l2k; a.l2k_n = t.l2k_n; a.l2v = t.l2v; a.l2v_n = t.l2v_n;
  a.k_signs = t.k_signs; a.cb3 = t.cb3; a.scale = t.scale; a.bias = t.summary_bias;
  a.agg = t.agg; a.Hkv = s.Hkv; a.G = s.G; a.ng = s.n_groups; a.beta = s.beta;
  a.want_topk = (mode & ROUTE_TOPK) ? 1 : 0;
  a.want_partial = (mode & ROUTE_PARTIALS) ? 1 : 0;
  a.given = a.want_topk ? nullptr : given;
  a.scores_out = scores_out;
  a.idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + w.idx_off);
  a.part = reinterpret_cast<float*>(ws + w.part_off);
  hipLaunchKernelGGL(summary_kernel<D>, dim3((unsigned)(s.B * s.Hkv)), dim3(kThreads),
                     summary_smem(D, s), st, a);
  return hipGetLastError();
}

hipError_t launch_route(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                        int mode, const int32_t* given, float* scores_out, int32_t* idx_out,
                        hipStream_t st) {
  if (s.n_groups == 0) return hipSuccess;
  if (!step_limits_ok(s)) return hipErrorInvalidValue;
  return s.d == 128 ? summary_d<128>(s, t, w, ws, mode, given, scores_out, idx_out, st)
                    : summary_d<64>(s, t, w, ws, mode, given, scores_out, idx_out, st);
}

template <int D>
hipError_t token_d(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                   const int32_t* idx, hipStream_t st) {
  TokArgs a{};
  a.q = t.q; a.l1k = t.l1k; a.l1k_n = t.l1k_n; a.l1v = t.l1v; a.l1v_n = t.l1v_n;
  a.l3 = t.l3; a.l3_staged = t.l3_staged; a.idx = idx;
  a.k_signs = t.k_signs; a.v_signs = t.v_signs; a.cb4 = t.cb4; a.scale = t.scale;
  a.Hkv = s.Hkv; a.G = s.G; a.n1 = s.n_l1; a.ng = s.n_groups; a.group_n = s.group_n;
  a.beta = s.beta;
  a.part = s.n_groups > 0 ? reinterpret_cast<const float*>(ws + w.part_off) : nullptr;
  a.out = t.out;
  hipLaunchKernelGGL(token_kernel<D>, dim3((unsigned)(s.B * s.Hkv)), dim3(kThreads),
                     token_smem(D, s), st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                       const int32_t* idx, hipStream_t st) {
  if (!step_limits_ok(s)) return hipErrorInvalidValue;
  return s.d == 128 ? token_d<128>(s, t, w, ws, idx, st) : token_d<64>(s, t, w, ws, idx, st);
}

}  // namespace hsq
