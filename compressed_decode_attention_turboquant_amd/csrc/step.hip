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
// Kernel R (route_kernel), one work-group per (unit, chunk of summary groups):
//   * 16 summaries per MFMA tile.  Summary keys are 3-bit; each lane turns
//     pairs of codes (6-bit fields) into fp16 pairs through an LDS table with
//     one copy per lane (no bank conflicts), split hi + lo so that
//     q_hi k_hi + q_hi k_lo + q_lo k_hi (three v_mfma_f32_16x16x32_f16) gives
//     fp32-accurate router scores.
//   * Query heads sit in the MFMA columns, each head twice (columns 2h, 2h+1):
//     the duplicate lets the value product run over (dim pair, token) with
//     k = 32, see below.  G <= 8 heads fill the 16 columns.
//   * router score = max (or mean) over the G heads; written per group.
//   * summary attention partial (online softmax) over the chunk.
//   * the last work-group of a unit (completion counter) selects the top-beta
//     groups (radix select on order-preserving keys, ties to the lower index,
//     output ascending) and adds a negative partial that removes the fetched
//     groups' summaries from the sum, so the masking needs no second pass.
// Kernel A (attn_kernel), one work-group per (unit, chunk of token tiles):
//   * 16 tokens per tile from L1 or from fetched L3 records; 4-bit codes go
//     through a byte -> fp16-pair table (one LDS copy per lane), QK and PV on
//     MFMA, online softmax in fp32.
//   * the last work-group of a unit merges all partials (log-sum-exp),
//     applies the inverse V rotation and writes the output.
//
// Value product layout.  O^T[dims][heads] = V^T P^T would need each lane to
// hold one dimension of several tokens, but codes are stored token-major.
// Instead the MFMA rows are dimension PAIRS and k runs over (token, e):
//     A[pair r][(n, e)] = V[n][2r + e],  B[(n, e)][(h, e')] = P[h][n] [e == e']
// so C[r][(h, e')] = O[h][2r + e'].  A lane then needs, per token, a byte (two
// 4-bit codes = two dims) straight from the token's code row, and B's columns
// (h, e') are exactly the duplicated-head columns of the QK output.
#include <cmath>

#include "hsq_device.h"
#include "hsq_internal.h"

namespace hsq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNC = 32;          // table copies: lanes l and l+32 share one (they are
                                 // served in different LDS passes, so no bank conflict)
constexpr int kMaxG = 8;
constexpr int kRouteWaves = 4;
constexpr int kAttnWaves = 8;
constexpr int kMaxGroups = 16384;  // top-beta keeps all scores of a unit in LDS
constexpr float kNegInf = -INFINITY;

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

// --------------------------------------------------------------- tables ----

// 4-bit: byte b (codes b & 15, b >> 4) -> fp16 pair, copy per lane.
__device__ void build_lut4(uint32_t* lut, const float* cb4, int tid, int nthr) {
  for (int i = tid; i < 256 * kNC; i += nthr) {
    const int e = i / kNC;
    lut[i] = h2u((_Float16)cb4[e & 15], (_Float16)cb4[e >> 4]);
  }
}

// 3-bit: 6-bit field e (codes e & 7, e >> 3) -> hi fp16 pair (table lut[0 ..
// 64*kNC)) and lo fp16 pair (lut[64*kNC ..)), with c = hi + lo to ~2^-22
// relative.  Two 4-byte tables: 8-byte LDS reads cost ~3.5x a 4-byte read.
__device__ void build_lut3(uint32_t* lut, const float* cb3, int tid, int nthr) {
  for (int i = tid; i < 64 * kNC; i += nthr) {
    const int e = i / kNC;
    const float c0 = cb3[e & 7], c1 = cb3[e >> 3];
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
    lut[i] = h2u(h0, h1);
    lut[64 * kNC + i] = h2u(l0, l1);
  }
}

__device__ __forceinline__ uint32_t lut4_at(const uint32_t* lut, uint32_t byte, int lane) {
  return lut[byte * kNC + (lane & (kNC - 1))];
}
__device__ __forceinline__ uint32_t lut3_hi(const uint32_t* lut, uint32_t e, int lane) {
  return lut[e * kNC + (lane & (kNC - 1))];
}
__device__ __forceinline__ uint32_t lut3_lo(const uint32_t* lut, uint32_t e, int lane) {
  return lut[64 * kNC + e * kNC + (lane & (kNC - 1))];
}

// ------------------------------------------------------- query rotation ----

// qf[h][i] = mult * (H D q_h)[i] for h < G, 0 for G <= h < 8.  Runs on the
// first 8*D/8 threads (whole waves).
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
// gq*D/4 + 8m + j for k-chunk m.  hi/lo fp16 split of the fp32 rotated query.
template <int D>
__device__ void query_operands(const float* qf, int lane, half8 (&hi)[D / 32], half8 (&lo)[D / 32]) {
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

// -------------------------------------------------------- tile products ----

// QK of 16 tokens with 4-bit keys.  kw: this lane's D/32 code dwords (token
// lane&15, dims gq*D/4 ..).  Returns S^T: rows = tokens 4gq+i, column = lane&15.
template <int D>
__device__ __forceinline__ f32x4 qk4(const uint32_t (&kw)[D / 32], const half8 (&qb)[D / 32],
                                     const uint32_t* lut, int lane) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const uint32_t w = kw[m];
    const half8 a = as_h8(lut4_at(lut, w & 0xffu, lane), lut4_at(lut, (w >> 8) & 0xffu, lane),
                          lut4_at(lut, (w >> 16) & 0xffu, lane), lut4_at(lut, w >> 24, lane));
    acc = mfma16(a, qb[m], acc);
  }
  return acc;
}

// 6-bit field at a compile-time bit position of a small word array.
template <int BIT>
__device__ __forceinline__ uint32_t field6(const uint32_t* w) {
  constexpr int k = BIT >> 5, s = BIT & 31;
  if constexpr (s <= 26) {
    return (w[k] >> s) & 63u;
  } else {
    return ((w[k] >> s) | (w[k + 1] << (32 - s))) & 63u;
  }
}

template <int D, int P>
__device__ __forceinline__ void lut3_pairs(const uint32_t* kw, const uint32_t* lut, int lane,
                                           uint32_t (&hi)[D / 8], uint32_t (&lo)[D / 8]) {
  if constexpr (P < D / 8) {
    const uint32_t e = field6<6 * P>(kw);
    hi[P] = lut3_hi(lut, e, lane);
    lo[P] = lut3_lo(lut, e, lane);
    lut3_pairs<D, P + 1>(kw, lut, lane, hi, lo);
  }
}

// QK of 16 summaries with 3-bit keys, three-term split product.
// kw: this lane's 3D/4 key bits (token lane&15, dims gq*D/4 ..) starting at bit 0.
template <int D>
__device__ __forceinline__ f32x4 qk3(const uint32_t (&kw)[3 * D / 128 + 1],
                                     const half8 (&qh)[D / 32], const half8 (&ql)[D / 32],
                                     const uint32_t* lut, int lane) {
  uint32_t hi[D / 8], lo[D / 8];
  lut3_pairs<D, 0>(kw, lut, lane, hi, lo);
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

// Load this lane's key bits of a 3-bit summary row (3D/8 bytes).
template <int D>
__device__ __forceinline__ void load_key3(const uint8_t* row, int gq, bool valid,
                                          uint32_t (&kw)[3 * D / 128 + 1]) {
  const uint32_t* r = reinterpret_cast<const uint32_t*>(row);
  if constexpr (D == 128) {  // 96 bits at dword 3*gq
    kw[0] = valid ? r[3 * gq] : 0u;
    kw[1] = valid ? r[3 * gq + 1] : 0u;
    kw[2] = valid ? r[3 * gq + 2] : 0u;
    kw[3] = 0u;
  } else {  // 48 bits at bit 48*gq: dwords (3gq)/2 and +1, shift 16*(gq&1)
    const int w = (3 * gq) >> 1;
    uint32_t a = valid ? r[w] : 0u, b = valid ? r[w + 1] : 0u;
    if (gq & 1) {
      a = (a >> 16) | (b << 16);
      b >>= 16;
    }
    kw[0] = a;
    kw[1] = b;
  }
}

// This lane's value bits of a 3-bit summary row: dims [2T*rho, 2T*rho + 2T)
// with T = D/32, i.e. 6T bits at bit 6T*rho, returned right-aligned.
template <int D>
__device__ __forceinline__ uint32_t load_val3(const uint8_t* row, int rho, bool valid) {
  if (!valid) return 0u;
  const uint32_t* r = reinterpret_cast<const uint32_t*>(row);
  constexpr int NW = 3 * D / 32;  // dwords per row
  const int bit = (6 * D / 32) * rho;
  const int w = bit >> 5, s = bit & 31;
  const uint32_t lo = r[w];
  const uint32_t hi = r[min(w + 1, NW - 1)];
  return s ? ((lo >> s) | (hi << (32 - s))) : lo;
}

// Value bits of a 4-bit token row for lane rho: bytes [T*rho, T*rho + T).
template <int D>
__device__ __forceinline__ uint32_t load_val4(const uint8_t* row, int rho, bool valid) {
  if (!valid) return 0u;
  if constexpr (D == 128) {
    return reinterpret_cast<const uint32_t*>(row)[rho];
  } else {
    return reinterpret_cast<const uint16_t*>(row)[rho];
  }
}

// PV product.  va[j]: value bits of token 4gq+j for this lane's row rho;
// p[j]: unnormalised weight (already times the value norm) of token 4gq+j for
// this lane's column (h, e').  O[t] accumulates O^T rows (pairs T*(4gq+i)+t).
template <int D, bool THREE>
__device__ __forceinline__ void pv(const uint32_t (&va)[4], const float (&p)[4], int lane,
                                   const uint32_t* lut4, const uint32_t* lut3, f32x4 (&O)[D / 32]) {
  constexpr int T = D / 32;
  const uint32_t sh = (lane & 1) ? 16u : 0u;
  uint32_t pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    pb[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p[j]) << sh;
  const half8 b = as_h8(pb[0], pb[1], pb[2], pb[3]);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    uint32_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (THREE)
        a[j] = lut3_hi(lut3, (va[j] >> (6 * t)) & 63u, lane);
      else
        a[j] = lut4_at(lut4, (va[j] >> (8 * t)) & 0xffu, lane);
    }
    O[t] = mfma16(as_h8(a[0], a[1], a[2], a[3]), b, O[t]);
  }
}

// ------------------------------------------------------ softmax state ----

template <int D>
struct Online {
  float m;   // running max of this lane's column (same on the 4 row-groups)
  float l;   // this lane's share of the denominator (4 rows)
  f32x4 O[D / 32];
  __device__ void init() {
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Fold in 4 logits of this lane (rows 4gq+i); returns the weights
  // exp(lg - m_new) scaled by sign (negative for removed entries).
  __device__ void update(const float (&lg)[4], float (&p)[4]) {
    float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float alpha = __expf(m - ms);
    l *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) O[t] *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __expf(lg[i] - ms);
    m = mn;
  }
};

// Combine the waves' states of a work-group and write one partial
// [m, l, O[0..D)] per head at dst (G heads).  scratch: kWaves*kMaxG*(D+2) floats.
template <int D, int WAVES>
__device__ void write_partial(const Online<D>& st, int G, float* scratch, float* dst, int tid) {
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
  for (int k = tid; k < G * (D + 2); k += WAVES * 64) {
    const int hh = k / (D + 2), e = k % (D + 2);
    float M = kNegInf;
    for (int v = 0; v < WAVES; ++v) M = fmaxf(M, scratch[(v * kMaxG + hh) * (D + 2)]);
    float acc = 0.f;
    for (int v = 0; v < WAVES; ++v) {
      const float* s = scratch + (v * kMaxG + hh) * (D + 2);
      if (e == 0) continue;
      const float wgt = (s[0] == kNegInf) ? 0.f : __expf(s[0] - M);
      acc += wgt * s[e];
    }
    dst[k] = (e == 0) ? M : acc;
  }
  __syncthreads();
}

// ------------------------------------------------------------- route ------

struct RouteArgs {
  const float* q;
  const uint8_t* l2k; const float* l2k_n; const uint8_t* l2v; const float* l2v_n;
  const uint32_t* k_signs; const float* cb3;
  float scale, bias;
  int agg, B, Hkv, G, ng, beta, chunks, tiles_per_chunk, mode;
  const int32_t* given;     // fetched set to mask (decode_attn), or null
  float* scores;            // [units][ng] workspace
  float* scores_out;        // optional user copy
  int32_t* idx;             // [units][beta] selection out (TOPK)
  float* part;              // partials
  int slots;                // partial slots per unit
  uint32_t* cnt;            // [units] completion counters
};

template <int D>
__device__ __forceinline__ void summary_tile(const RouteArgs& a, int unit, const int32_t* gid,
                                             int g0, int gend, bool negative,
                                             const uint32_t* fetched_mask, const half8 (&qh)[D / 32],
                                             const half8 (&ql)[D / 32], const uint32_t* lut3,
                                             int lane, Online<D>& st, bool want_agg) {
  constexpr int CB3 = 3 * D / 8;
  const int n = lane & 15, gq = lane >> 4, c = lane & 15;
  // key rows: token n of the tile
  const int gn = g0 + n;
  const bool vn = gn < gend;
  const int grow = vn ? (gid ? gid[gn] : gn) : 0;
  uint32_t kw[3 * D / 128 + 1];
  load_key3<D>(a.l2k + ((size_t)unit * a.ng + grow) * CB3, gq, vn, kw);
  const f32x4 acc = qk3<D>(kw, qh, ql, lut3, lane);
  float s[4], lg[4], p[4];
  int gr[4];
  bool vr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gi = g0 + 4 * gq + i;
    vr[i] = gi < gend;
    gr[i] = vr[i] ? (gid ? gid[gi] : gi) : 0;
    const float rk = vr[i] ? a.l2k_n[(size_t)unit * a.ng + gr[i]] : 0.f;
    s[i] = vr[i] ? acc[i] * rk : kNegInf;
  }
  if (want_agg) {
    const int G2 = 2 * a.G;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v;
      if (a.agg == HSQ_AGG_MAX) {
        v = (c < G2) ? s[i] : kNegInf;
        v = fmaxf(v, __shfl_xor(v, 1, 64));
        v = fmaxf(v, __shfl_xor(v, 2, 64));
        v = fmaxf(v, __shfl_xor(v, 4, 64));
        v = fmaxf(v, __shfl_xor(v, 8, 64));
      } else {
        v = (c < G2 && vr[i]) ? s[i] : 0.f;
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 8, 64);
        v = v / (float)G2;
      }
      if (c == i && vr[i]) {
        a.scores[(size_t)unit * a.ng + gr[i]] = v;
        if (a.scores_out) a.scores_out[(size_t)unit * a.ng + gr[i]] = v;
      }
    }
  }
  if (a.mode & ROUTE_PARTIALS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bool live = vr[i];
      if (fetched_mask && live) live = !((fetched_mask[gr[i] >> 5] >> (gr[i] & 31)) & 1u);
      lg[i] = live ? s[i] + a.bias : kNegInf;
    }
    st.update(lg, p);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float rv = vr[i] ? a.l2v_n[(size_t)unit * a.ng + gr[i]] : 0.f;
      psum += p[i];
      p[i] = (negative ? -p[i] : p[i]) * rv;
    }
    st.l += negative ? -psum : psum;
    // value rows: lane rho = lane&15 takes its bits of tokens 4gq+j
    uint32_t va[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gj = g0 + 4 * gq + j;
      const bool vj = gj < gend;
      const int rj = vj ? (gid ? gid[gj] : gj) : 0;
      va[j] = load_val3<D>(a.l2v + ((size_t)unit * a.ng + rj) * CB3, n, vj);
    }
    pv<D, true>(va, p, lane, nullptr, lut3, st.O);
  }
}

// Ordered uint32 key of a float: larger float <-> larger key.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the work-group (WAVES*64 threads).
template <int WAVES>
__device__ int block_exclusive_scan(int v, int* tmp, int tid, int& total) {
  const int lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < WAVES; ++w) {
    if (w < wave) base += tmp[w];
    tot += tmp[w];
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// Top-beta of the unit's scores: sel[0..beta) ascending group ids.
template <int WAVES>
__device__ void top_beta(const float* scores, int ng, int beta, uint32_t* keys, int* hist,
                         int* tmp, int32_t* sel, int tid) {
  constexpr int NT = WAVES * 64;
  if (beta <= 0) return;
  if (beta >= ng) {
    for (int g = tid; g < ng; g += NT) sel[g] = g;
    __syncthreads();
    return;
  }
  for (int g = tid; g < ng; g += NT) keys[g] = fkey(scores[g]);
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_need;
  if (tid == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_need = beta;
  }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += NT) hist[b] = 0;
    __syncthreads();
    const uint32_t pre = s_prefix, msk = s_mask;
    for (int g = tid; g < ng; g += NT) {
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
      const bool here = excl < need && incl >= need;
      if (here) {
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
  const int ties_needed = s_need;  // number of keys equal to kth to take
  // contiguous ranges per thread keep index order
  const int per = (ng + NT - 1) / NT;
  const int lo = min(tid * per, ng), hi = min(lo + per, ng);
  int n_eq = 0;
  for (int g = lo; g < hi; ++g) n_eq += keys[g] == kth;
  int tot;
  const int eq_base = block_exclusive_scan<WAVES>(n_eq, tmp, tid, tot);
  int n_sel = 0, e = eq_base;
  for (int g = lo; g < hi; ++g) {
    const uint32_t k = keys[g];
    if (k > kth) ++n_sel;
    else if (k == kth) n_sel += (e++ < ties_needed);
  }
  const int sel_base = block_exclusive_scan<WAVES>(n_sel, tmp, tid, tot);
  int pos = sel_base;
  e = eq_base;
  for (int g = lo; g < hi; ++g) {
    const uint32_t k = keys[g];
    bool take = k > kth;
    if (k == kth) take = (e++ < ties_needed);
    if (take) sel[pos++] = g;
  }
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(RouteArgs a) {
  extern __shared__ __align__(16) char smem[];
  uint32_t* lut3 = reinterpret_cast<uint32_t*>(smem);
  float* qf = reinterpret_cast<float*>(smem + 64 * kNC * 8);
  char* scr = reinterpret_cast<char*>(qf + kMaxG * D);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x / a.chunks, chunk = blockIdx.x % a.chunks;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;

  build_lut3(lut3, a.cb3, tid, kRouteWaves * 64);
  rotate_queries<D>(a.q + ((size_t)b * a.Hkv + kvh) * a.G * D, a.k_signs + kvh * (D / 32), a.G,
                    a.scale * rsqrtf((float)D), qf, tid);
  uint32_t* fmask = nullptr;
  if (a.given) {  // fetched-set bitmap for direct masking
    fmask = reinterpret_cast<uint32_t*>(scr);
    const int words = (a.ng + 31) / 32;
    for (int w = tid; w < words; w += kRouteWaves * 64) fmask[w] = 0u;
    __syncthreads();
    for (int i = tid; i < a.beta; i += kRouteWaves * 64) {
      const int g = a.given[(size_t)unit * a.beta + i];
      if (g >= 0 && g < a.ng) atomicOr(&fmask[g >> 5], 1u << (g & 31));
    }
  }
  __syncthreads();
  half8 qh[D / 32], ql[D / 32];
  query_operands<D>(qf, lane, qh, ql);

  Online<D> st;
  st.init();
  const int n_tiles = (a.ng + 15) / 16;
  const int t0 = chunk * a.tiles_per_chunk;
  const int t1 = min(t0 + a.tiles_per_chunk, n_tiles);
  const bool agg = (a.mode & ROUTE_TOPK) != 0;
  for (int t = t0 + wave; t < t1; t += kRouteWaves)
    summary_tile<D>(a, unit, nullptr, t * 16, a.ng, false, fmask, qh, ql, lut3, lane, st, agg);

  float* scratch = reinterpret_cast<float*>(scr + (a.given ? ((a.ng + 31) / 32 * 4 + 15) / 16 * 16 : 0));
  if (a.mode & ROUTE_PARTIALS)
    write_partial<D, kRouteWaves>(st, a.G, scratch,
                                  a.part + ((size_t)unit * a.slots + chunk) * a.G * (D + 2), tid);
  if (!(a.mode & ROUTE_TOPK)) {
    // given-set mode: slot `chunks` stays an empty partial
    if ((a.mode & ROUTE_PARTIALS) && chunk == 0) {
      float* e = a.part + ((size_t)unit * a.slots + a.chunks) * a.G * (D + 2);
      for (int k = tid; k < a.G * (D + 2); k += kRouteWaves * 64)
        e[k] = (k % (D + 2) == 0) ? kNegInf : 0.f;
    }
    return;
  }

  // ---- completion counter: the last chunk of the unit selects top-beta ----
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&a.cnt[unit], 1u) == (uint32_t)(a.chunks - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  uint32_t* keys = reinterpret_cast<uint32_t*>(scr);
  int* hist = reinterpret_cast<int*>(keys + a.ng);
  int* tmp = hist + 256;
  int32_t* sel = tmp + 16;
  const float* sc = a.scores + (size_t)unit * a.ng;
  top_beta<kRouteWaves>(sc, a.ng, a.beta, keys, hist, tmp, sel, tid);
  for (int i = tid; i < a.beta; i += kRouteWaves * 64) a.idx[(size_t)unit * a.beta + i] = sel[i];
  if (a.mode & ROUTE_PARTIALS) {
    // negative partial over the fetched summaries: removes them from the sum
    Online<D> neg;
    neg.init();
    const int nt = (a.beta + 15) / 16;
    for (int t = wave; t < nt; t += kRouteWaves)
      summary_tile<D>(a, unit, sel, t * 16, a.beta, true, nullptr, qh, ql, lut3, lane, neg, false);
    float* scratch2 = reinterpret_cast<float*>(
        reinterpret_cast<char*>(sel) + ((size_t)a.beta * 4 + 15) / 16 * 16);
    write_partial<D, kRouteWaves>(neg, a.G, scratch2,
                                  a.part + ((size_t)unit * a.slots + a.chunks) * a.G * (D + 2), tid);
  }
  if (tid == 0) a.cnt[unit] = 0u;
}

// ------------------------------------------------------------ attention ---

struct AttnArgs {
  const float* q;
  const uint8_t* l1k; const float* l1k_n; const uint8_t* l1v; const float* l1v_n;
  const uint8_t* l3; int l3_staged;
  const int32_t* idx;
  const uint32_t* k_signs; const uint32_t* v_signs; const float* cb4;
  float scale;
  int B, Hkv, G, n1, ng, group_n, beta, chunks, tiles_per_chunk;
  float* part;
  int r_slots, slots;
  uint32_t* cnt;
  float* out;
};

template <int D>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_kernel(AttnArgs a) {
  constexpr int CB = D / 2;
  constexpr int NW = kAttnWaves * 64;
  extern __shared__ __align__(16) char smem[];
  uint32_t* lut4 = reinterpret_cast<uint32_t*>(smem);
  float* qf = reinterpret_cast<float*>(smem + 256 * kNC * 4);
  float* scratch = qf + kMaxG * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x / a.chunks, chunk = blockIdx.x % a.chunks;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int n = lane & 15, gq = lane >> 4;

  build_lut4(lut4, a.cb4, tid, NW);
  rotate_queries<D>(a.q + ((size_t)b * a.Hkv + kvh) * a.G * D, a.k_signs + kvh * (D / 32), a.G,
                    a.scale * rsqrtf((float)D), qf, tid);
  __syncthreads();
  half8 qh[D / 32], ql[D / 32];
  query_operands<D>(qf, lane, qh, ql);

  const int n1t = (a.n1 + 15) / 16;
  const int nft = (a.group_n == 16) ? a.beta : (a.beta + 1) / 2;
  const int total = n1t + nft;
  const int t0 = chunk * a.tiles_per_chunk;
  const int t1 = min(t0 + a.tiles_per_chunk, total);
  const size_t rec = (size_t)a.group_n * (D + 8);

  Online<D> st;
  st.init();
  for (int t = t0 + wave; t < t1; t += kAttnWaves) {
    // row pointers for token row r of this tile
    auto rows = [&](int r, const uint8_t*& kr, const float*& kn, const uint8_t*& vr,
                    const float*& vn) -> bool {
      if (t < n1t) {
        const int tok = t * 16 + r;
        if (tok >= a.n1) return false;
        const size_t o = (size_t)unit * a.n1 + tok;
        kr = a.l1k + o * CB; kn = a.l1k_n + o; vr = a.l1v + o * CB; vn = a.l1v_n + o;
        return true;
      }
      const int f = t - n1t;
      const int slot = (a.group_n == 16) ? f : 2 * f + (r >> 3);
      const int tok = (a.group_n == 16) ? r : (r & 7);
      if (slot >= a.beta) return false;
      const uint8_t* base;
      if (a.l3_staged) {
        base = a.l3 + ((size_t)unit * a.beta + slot) * rec;
      } else {
        const int g = a.idx[(size_t)unit * a.beta + slot];
        if (g < 0 || g >= a.ng) return false;  // invalid id: the slot is skipped
        base = a.l3 + ((size_t)unit * a.ng + g) * rec;
      }
      const int N = a.group_n;
      kr = base + (size_t)tok * CB;
      kn = reinterpret_cast<const float*>(base + (size_t)N * CB) + tok;
      vr = base + (size_t)N * (CB + 4) + (size_t)tok * CB;
      vn = reinterpret_cast<const float*>(base + (size_t)N * (2 * CB + 4)) + tok;
      return true;
    };
    const uint8_t *kr, *vr;
    const float *kn, *vn;
    // keys: lane row n
    uint32_t kw[D / 32];
    {
      const bool ok = rows(n, kr, kn, vr, vn);
      const uint32_t* p = reinterpret_cast<const uint32_t*>(kr + gq * (D / 8));
#pragma unroll
      for (int m = 0; m < D / 32; ++m) kw[m] = ok ? p[m] : 0u;
    }
    const f32x4 acc = qk4<D>(kw, qh, lut4, lane);
    float lg[4], p[4], rvs[4];
    uint32_t va[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = rows(4 * gq + i, kr, kn, vr, vn);
      lg[i] = ok ? acc[i] * kn[0] : kNegInf;
      rvs[i] = ok ? vn[0] : 0.f;
      va[i] = load_val4<D>(vr, n, ok);
    }
    st.update(lg, p);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      psum += p[i];
      p[i] *= rvs[i];
    }
    st.l += psum;
    pv<D, false>(va, p, lane, lut4, nullptr, st.O);
  }
  write_partial<D, kAttnWaves>(st, a.G, scratch,
                               a.part + ((size_t)unit * a.slots + a.r_slots + chunk) * a.G * (D + 2),
                               tid);

  // ---- the last chunk of the unit merges every partial ----
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&a.cnt[unit], 1u) == (uint32_t)(a.chunks - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* pu = a.part + (size_t)unit * a.slots * a.G * (D + 2);
  float* o = scratch;  // [G][D] merged, normalised, rotated domain
  for (int k = tid; k < a.G * D; k += NW) {
    const int h = k / D, e = k % D;
    float M = kNegInf;
    for (int s = 0; s < a.slots; ++s) M = fmaxf(M, pu[((size_t)s * a.G + h) * (D + 2)]);
    float L = 0.f, acc2 = 0.f;
    for (int s = 0; s < a.slots; ++s) {
      const float* ps = pu + ((size_t)s * a.G + h) * (D + 2);
      const float w = (ps[0] == kNegInf) ? 0.f : __expf(ps[0] - M);
      L += w * ps[1];
      acc2 += w * ps[2 + e];
    }
    o[k] = (L > 0.f) ? acc2 / L : 0.f;
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
      float* dst = a.out + (((size_t)b * a.Hkv + kvh) * a.G + h) * D + 8 * sub;
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = flip(v[k] * sc, (sb >> k) & 1u);
    }
  }
  if (tid == 0) a.cnt[unit] = 0u;
}

int chunks_for(int units, int tiles, int per_wave_min, int waves) {
  // enough work-groups to fill 256 CUs a few times over, but at least
  // per_wave_min tiles per wave
  const int want = (4 * 256 + units - 1) / units;
  const int cap = std::max(1, tiles / std::max(1, per_wave_min * waves));
  return std::max(1, std::min(want, cap));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t route_smem(int D, const StepShape& s, bool given) {
  size_t base = 64 * kNC * 8 + kMaxG * D * 4;
  const size_t mask = given ? ((size_t)(s.n_groups + 31) / 32 * 4 + 15) / 16 * 16 : 0;
  const size_t comb = (size_t)kRouteWaves * kMaxG * (D + 2) * 4;
  const size_t topk = (size_t)s.n_groups * 4 + 256 * 4 + 16 * 4 + ((size_t)s.beta * 4 + 15) / 16 * 16 + comb;
  return base + std::max(mask + comb, topk);
}

size_t attn_smem(int D) {
  return 256 * kNC * 4 + kMaxG * D * 4 + (size_t)kAttnWaves * kMaxG * (D + 2) * 4;
}

}  // namespace

Workspace plan_workspace(const StepShape& s) {
  Workspace w{};
  const int units = s.B * s.Hkv;
  const int r_tiles = (s.n_groups + 15) / 16;
  w.route_chunks = s.n_groups > 0 ? chunks_for(units, r_tiles, 2, kRouteWaves) : 0;
  const int n1t = (s.n_l1 + 15) / 16;
  const int nft = (s.group_n == 16) ? s.beta : (s.beta + 1) / 2;
  w.fetch_chunks = chunks_for(units, n1t + nft, 2, kAttnWaves);
  w.attn_slots = (w.route_chunks ? w.route_chunks + 1 : 0) + w.fetch_chunks;
  size_t off = 0;
  w.scores_off = off; off = align256(off + (size_t)units * std::max(s.n_groups, 1) * 4);
  w.idx_off = off;    off = align256(off + (size_t)units * std::max(s.beta, 1) * 4);
  w.part_off = off;   off = align256(off + (size_t)units * w.attn_slots * s.G * (s.d + 2) * 4);
  w.cnt_off = off;    off = align256(off + (size_t)units * 2 * 4);
  w.qrot_off = 0;
  w.total = off;
  return w;
}

hipError_t launch_qrot(const StepShape&, const StepTensors&, const Workspace&, char*, hipStream_t) {
  return hipSuccess;  // the query rotation runs inside both kernels' prologue
}

template <int D>
hipError_t route_d(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                   int mode, const int32_t* given, float* scores_out, int32_t* idx_out,
                   hipStream_t st) {
  RouteArgs a{};
  a.q = t.q; a.l2k = t.l2k; a.l2k_n = t.l2k_n; a.l2v = t.l2v; a.l2v_n = t.l2v_n;
  a.k_signs = t.k_signs; a.cb3 = t.cb3; a.scale = t.scale; a.bias = t.summary_bias;
  a.agg = t.agg; a.B = s.B; a.Hkv = s.Hkv; a.G = s.G; a.ng = s.n_groups; a.beta = s.beta;
  a.chunks = w.route_chunks;
  a.tiles_per_chunk = ((s.n_groups + 15) / 16 + a.chunks - 1) / a.chunks;
  a.mode = mode;
  a.given = (mode & ROUTE_TOPK) ? nullptr : given;
  a.scores = reinterpret_cast<float*>(ws + w.scores_off);
  a.scores_out = scores_out;
  a.idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + w.idx_off);
  a.part = reinterpret_cast<float*>(ws + w.part_off);
  a.slots = w.attn_slots;
  a.cnt = reinterpret_cast<uint32_t*>(ws + w.cnt_off);
  const size_t smem = route_smem(D, s, a.given != nullptr);
  const unsigned grid = (unsigned)(s.B * s.Hkv * a.chunks);
  hipLaunchKernelGGL(route_kernel<D>, dim3(grid), dim3(kRouteWaves * 64), smem, st, a);
  return hipGetLastError();
}

hipError_t launch_route(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                        int mode, const int32_t* given, float* scores_out, int32_t* idx_out,
                        hipStream_t st) {
  if (s.n_groups == 0) return hipSuccess;
  if (s.n_groups > kMaxGroups) return hipErrorInvalidValue;
  return s.d == 128 ? route_d<128>(s, t, w, ws, mode, given, scores_out, idx_out, st)
                    : route_d<64>(s, t, w, ws, mode, given, scores_out, idx_out, st);
}

template <int D>
hipError_t attn_d(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                  const int32_t* idx, hipStream_t st) {
  AttnArgs a{};
  a.q = t.q; a.l1k = t.l1k; a.l1k_n = t.l1k_n; a.l1v = t.l1v; a.l1v_n = t.l1v_n;
  a.l3 = t.l3; a.l3_staged = t.l3_staged; a.idx = idx;
  a.k_signs = t.k_signs; a.v_signs = t.v_signs; a.cb4 = t.cb4; a.scale = t.scale;
  a.B = s.B; a.Hkv = s.Hkv; a.G = s.G; a.n1 = s.n_l1; a.ng = s.n_groups; a.group_n = s.group_n;
  a.beta = s.beta; a.chunks = w.fetch_chunks;
  const int n1t = (s.n_l1 + 15) / 16;
  const int nft = (s.group_n == 16) ? s.beta : (s.beta + 1) / 2;
  a.tiles_per_chunk = (n1t + nft + a.chunks - 1) / a.chunks;
  a.part = reinterpret_cast<float*>(ws + w.part_off);
  a.r_slots = w.route_chunks ? w.route_chunks + 1 : 0;
  a.slots = w.attn_slots;
  a.cnt = reinterpret_cast<uint32_t*>(ws + w.cnt_off) + s.B * s.Hkv;
  a.out = t.out;
  const unsigned grid = (unsigned)(s.B * s.Hkv * a.chunks);
  hipLaunchKernelGGL(attn_kernel<D>, dim3(grid), dim3(kAttnWaves * 64), attn_smem(D), st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                       const int32_t* idx, hipStream_t st) {
  return s.d == 128 ? attn_d<128>(s, t, w, ws, idx, st) : attn_d<64>(s, t, w, ws, idx, st);
}

}  // namespace hsq
