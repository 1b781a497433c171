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
//                   tile, codes turned into exact fp16 centroid pairs through
//                   a lane-replicated LDS table; the query split q_hi + q_lo
//                   (two v_mfma_f32_16x16x32_f16) gives fp32-accurate scores;
//                   the per-head logits stay in LDS.  (2)+(3) every wave
//                   streams the values of ALL summaries into the softmax
//                   partial (each head's maximum logit is known from (1)),
//                   while the router scores (max or mean over the G heads) and
//                   the exact top-beta (score histogram, then an exact ranking
//                   of the threshold bucket) run in steps between segments of
//                   that stream; finally the fetched summaries are subtracted
//                   with the same weights and dequantised values.  One partial
//                   per unit.
//   token_kernel    16 tokens per tile from L1 and from the fetched L3 records;
//                   4-bit codes through a byte -> fp16-pair table (one LDS copy
//                   per lane, address built by one v_perm); QK and PV on MFMA;
//                   merge with the summary partial (log-sum-exp); inverse V
//                   rotation; output.
// Loads go through buffer descriptors scoped to the unit, so rows past the end
// and masked rows read as zero without touching memory, and the tile loops
// need no per-lane branches.  Each wave keeps two tiles' loads in flight while
// it computes the current one; work-group barriers wait for LDS traffic only,
// so those loads stay in flight across them.
//
// Value product layout.  O^T[dims][heads] = V^T P^T would need each lane to
// hold one dimension of several tokens, but codes are stored token-major.
// Instead the MFMA rows are dimension PAIRS and k runs over (token, e):
//     A[pair r][(n, e)] = V[n][2r + e],  B[(n, e)][(h, e')] = P[h][n] [e == e']
// so C[r][(h, e')] = O[h][2r + e'].  A lane then needs, per token, a byte (two
// 4-bit codes = two dims) straight from the token's code row, and B's columns
// are exactly the QK output columns when each head's query is placed in two
// columns: column c holds (h, e') = (c & 7, c >> 3).  G <= 8 heads fill the 16
// columns.
#include <cmath>
#include <type_traits>

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
constexpr int kLut4Bytes = 256 * kNC4 * 4;  // 4-bit table of the two-launch kernels
constexpr int kMaxGroups = 16384;
constexpr int kMaxLogits = 12288;        // G * n_groups kept in LDS (one-launch step, route)
constexpr int kSplitUnits = 128;         // fewer units than this: the split step
constexpr size_t kMaxFusedLds = 92 * 1024;  // dynamic LDS of the one-launch step (64 KB static)
constexpr uint32_t kFar = 0x80000000u;   // buffer offset that reads as zero
constexpr float kNegInf = -INFINITY;
constexpr float kPosInf = INFINITY;
// tiles per wave in the load pipelines (K-1 in flight while one computes);
// measured best on the 16K-context headline layer (deeper value pipelines
// lengthen the segments between the selection steps; the token tiles are
// held to 3 by the register budget)
constexpr int kKeyDepth = 4;
constexpr int kValDepth = 4;
constexpr int kTokDepth = 3;

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
// Four consecutive floats in one 16-byte load.  The buffer range check is
// made per dword, so a load that crosses the end of the buffer returns the
// floats in range and zeros past the end (the ragged-tail parity tests cover
// this); the tile loads need no edge case, and every path through a
// pipelined loop issues the same loads, which keeps the waits exact.
__device__ __forceinline__ f32x4 ldf4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, ld128(r, off));
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
// Row norms.  Lane (c, gq) handles rows 4gq .. 4gq+3 of a tile and loads the
// norm of row 4gq + (c & 3) only; lane c & 3 == i of each quad then holds row
// 4gq + i, so quad_perm [i,i,i,i] gives every lane row i's norm, and the DPP
// move fuses into the multiply that uses it (one register per tile, not four).
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), I * 0x55, 0xf, 0xf, true));
}
__device__ __forceinline__ f32x4 mul_rows(f32x4 a, float nrm) {
  return f32x4{a[0] * quad_bcast<0>(nrm), a[1] * quad_bcast<1>(nrm), a[2] * quad_bcast<2>(nrm),
               a[3] * quad_bcast<3>(nrm)};
}
__device__ __forceinline__ float row_norm(float nrm, int r) {
  return r == 0 ? quad_bcast<0>(nrm)
                : (r == 1 ? quad_bcast<1>(nrm) : (r == 2 ? quad_bcast<2>(nrm) : quad_bcast<3>(nrm)));
}

// Runs use(i, B[i % K]) for i in [0, iters) with each buffer's loads
// issued K-1 iterations before its use, so every wave keeps K-1 tiles in
// flight while it computes one.  The uses run in segments: [K*q0, K*q1) of a
// run of `iters` (q0, q1 counted in K-tuples), so that other work can go
// between segments while the loads issued at the end of one are in flight.
// On entry B[0..K-2] hold (or are loading) tiles K*q0 .. K*q0+K-2; on exit
// the tiles K*q1 .. K*q1+K-2.  load(i) is also called for i >= iters; it must
// then read out of bounds (buffer loads past num_records return zero without
// memory traffic).  iters is wave-uniform.
//
// Every pass issues all K loads, so the number of loads in flight is the same
// on every path through the body and the waits stay partial; the trailing
// uses are skipped by wave-uniform tests instead of a second copy of the
// body.  The scheduling barriers keep the compiler from sinking the loads
// below the previous tile's arithmetic.
template <int K, typename Buf, typename LoadF, typename UseF>
__device__ __forceinline__ void pipeline_seg(int q0, int q1, int iters, Buf (&B)[K], LoadF load,
                                             UseF use) {
  for (int i = K * q0; i < K * q1; i += K) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      load(i + j + K - 1, B[(j + K - 1) % K]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + j < iters) use(i + j, B[j]);
    }
  }
}
// The whole run in one segment.
template <int K, typename Buf, typename LoadF, typename UseF>
__device__ __forceinline__ void pipeline(int iters, Buf (&B)[K], LoadF load, UseF use) {
  pipeline_seg<K>(0, (iters + K - 1) / K, iters, B, load, use);
}

// Lane index, read afresh at each use (the asm is volatile, so the
// compiler neither hoists nor keeps it): the per-lane parts of the tile
// addresses are a few VALU from it, cheaper than registers held across a
// loop or spilled (a reload waits for every load in flight).
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
// Wave index as a scalar (wave-uniform for the compiler).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
template <int NW = kWaves>
__device__ __forceinline__ int wave_iters(int n_tiles, int wave) {
  return wave < n_tiles ? (n_tiles - wave + NW - 1) / NW : 0;
}

// Skewed split of n tiles over NW waves.  Where two waves share a SIMD the
// older one gets the issue slots first, so the waves of the first half of a
// work-group run a tile in less time than those of the second half (about
// 1.2 against 1.45 us in the headline stream).  Every wave takes tiles
// w, w + NW, .. for m = n / 8.4 rounds; the tiles after those go to the first
// half only (NW m + w + NW/2 j): with 127 tiles, 15 a wave in the second
// half and 16-17 in the first.  Indices past a wave's own tiles are out of
// range (they load zeros), so the pipelines' look-ahead reads nothing.
// (Measured on the headline stream: 57.4 -> 57.0 us; splits of n / 8.8 and
// n / 9.5 rounds gained less.)
template <int NW, int K>
__device__ __forceinline__ int skew_rounds(int n) {
  return max(K - 1, min((n + NW - 1) / NW, n * 10 / 84));
}
template <int NW>
__device__ __forceinline__ int skew_tile(int i, int m, int w, int n) {
  if (i < m) return w + NW * i;
  return w < NW / 2 ? NW * m + w + (NW / 2) * (i - m) : n + NW * (i - m + 1);
}
template <int NW>
__device__ __forceinline__ int skew_iters(int n, int m, int w) {
  const int common = w < n ? min(m, (n - w + NW - 1) / NW) : 0;
  if (w >= NW / 2) return common;
  const int rest = n - NW * m - w;
  return common + (rest > 0 ? (rest + NW / 2 - 1) / (NW / 2) : 0);
}

// Wave-wide maximum / minimum by DPP row operations (GFX9 row broadcasts);
// the result is read from the last lane, so it is wave-uniform.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float x) {
  const int v = __float_as_int(x);
  return __int_as_float(__builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xb1>(x));        // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_f<0x4e>(x));        // quad_perm 2,3,0,1
  x = fmaxf(x, dpp_f<0x141>(x));       // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));       // row_mirror
  x = fmaxf(x, dpp_f<0x142, 0xa>(x));  // row_bcast:15
  x = fmaxf(x, dpp_f<0x143, 0xc>(x));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_min(float x) { return -wave_max(-x); }
// Wave-wide unsigned minimum / maximum by the same DPP steps (no LDS
// traffic); wave-uniform result.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  x = min(x, dpp_u<0xb1>(x));
  x = min(x, dpp_u<0x4e>(x));
  x = min(x, dpp_u<0x141>(x));
  x = min(x, dpp_u<0x140>(x));
  x = min(x, dpp_u<0x142, 0xa>(x));
  x = min(x, dpp_u<0x143, 0xc>(x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = max(x, dpp_u<0xb1>(x));
  x = max(x, dpp_u<0x4e>(x));
  x = max(x, dpp_u<0x141>(x));
  x = max(x, dpp_u<0x140>(x));
  x = max(x, dpp_u<0x142, 0xa>(x));
  x = max(x, dpp_u<0x143, 0xc>(x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
// Inclusive prefix sum over the lanes of a wave by DPP steps (no LDS
// traffic): row shifts by 1, 2, 4, 8 sum each row of 16 lanes, then the row
// broadcasts of lanes 15 and 31 carry the totals of the lower rows.  A lane
// whose source is outside its row, or whose row is masked off, adds 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_z(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_z<0x111>(x);       // row_shr:1
  x += dpp_z<0x112>(x);       // row_shr:2
  x += dpp_z<0x114>(x);       // row_shr:4
  x += dpp_z<0x118>(x);       // row_shr:8
  x += dpp_z<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_z<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
// Sum over aligned groups of LANES (8 or 16) consecutive lanes by DPP row
// operations; every lane of a group gets its group's sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 8 || LANES == 16, "8 or 16 lanes");
  x += dpp_f<0xb1>(x);   // quad_perm 1,0,3,2
  x += dpp_f<0x4e>(x);   // quad_perm 2,3,0,1
  x += dpp_f<0x141>(x);  // row_half_mirror: the other quad of the half row
  if constexpr (LANES == 16) x += dpp_f<0x140>(x);  // row_mirror: the other half
  return x;
}

// Three-way minimum / maximum as one VALU instruction.  fminf/fmaxf would
// first quiet every operand the compiler cannot prove canonical (one more
// instruction each); the bounds below only need an order, and a NaN operand
// is dropped by the instruction itself.
__device__ __forceinline__ float min3f(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// ---------------------------------------------------------------- tables ---
//
// The dequantisation tables live in static LDS, so their base folds into the
// ds_read offset field and a lookup costs one address instruction.

// 4-bit: byte b (codes b & 15, b >> 4) -> fp16 pair; copy l at dword b*64 + l,
// so lane l's address is (b << 8) | (l << 2): one v_perm from the code dword.
__device__ void build_lut4(uint32_t* lut, const float* cb, int tid) {
  // 16-byte chunk c holds copies 4(c%16) .. 4(c%16)+3 of entry c/16; thread t
  // writes chunks t, t + 512, ..., so the lanes of a wave write consecutive
  // chunks (a write per entry and lane pair would put every even lane of a
  // wave on the same four banks)
  u32x4* dst = reinterpret_cast<u32x4*>(lut);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = k * kThreads + tid;
    const int e = c >> 4;
    const uint32_t v = h2u((_Float16)cb[e & 15], (_Float16)cb[e >> 4]);
    dst[c] = u32x4{v, v, v, v};
  }
}
// byte K of w as a table address for this lane
template <int K>
__device__ __forceinline__ uint32_t lut4_addr(uint32_t w, uint32_t lane4) {
  // bytes of {lane4 (sel 4..7), w (sel 0..3)}: result = [lane4.b0, w.bK, 0, 0]
  return __builtin_amdgcn_perm(lane4, w, 0x0c0c0004u | (uint32_t(K) << 8));
}
__device__ __forceinline__ uint32_t lds_at(const uint32_t* base, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + byte_addr);
}

// 3-bit: 6-bit field e (codes e & 7, e >> 3) -> fp16 pair at dword e*32 + l%32
// (the stored fp32 centroids rounded to the nearest fp16).
__device__ void build_lut3(uint32_t* lut, const float* cb, int tid) {
  // thread t fills copies 4(t&7) .. 4(t&7)+3 of entry t/8
  const int e = tid >> 3;
  const uint32_t v = h2u((_Float16)cb[e & 7], (_Float16)cb[e >> 3]);
  *reinterpret_cast<u32x4*>(lut + e * kNC3 + 4 * (tid & 7)) = u32x4{v, v, v, v};
}
// 3-bit low parts for the exact router: entry e holds the fp16 pair of
// kLoScale * (c - fp16(c)) for codes e & 7, e >> 3 (scaled so that the parts
// stay normal fp16 numbers); hi + lo / kLoScale = c to about 2^-23 relative.
constexpr float kLoScale = 4096.f;
__device__ void build_lut3_lo(uint32_t* lut, const float* cb, int tid) {
  const int e = tid >> 3;
  const float c0 = cb[e & 7], c1 = cb[e >> 3];
  const uint32_t v = h2u((_Float16)((c0 - (float)(_Float16)c0) * kLoScale),
                         (_Float16)((c1 - (float)(_Float16)c1) * kLoScale));
  *reinterpret_cast<u32x4*>(lut + e * kNC3 + 4 * (tid & 7)) = u32x4{v, v, v, v};
}
// table address of 6-bit field e for this lane (lane4 = (lane & 31) << 2)
__device__ __forceinline__ uint32_t lut3_addr(uint32_t e, uint32_t lane4) {
  return (e << 7) | lane4;
}

// Columns of the MFMA products.  Column c of a QK or PV tile belongs to
// head c & 7 and, in the value products, to element c >> 3 of each
// dimension pair; so columns c and c + 8 carry the same head, and the two
// halves of the router's query split (columns h and h + 8) add up by one row
// rotation into a value that both columns then hold.
__device__ __forceinline__ int col_head(int c) { return c & 7; }
__device__ __forceinline__ int col_elem(int c) { return c >> 3; }

// -------------------------------------------------------- query rotation ---

// Query rotation in two steps so that its global loads can be issued with
// the first tile loads: load_query, then rotate_query writes
// qf[h*QS + i] = mult * (H D q_h)[i] for h < G and 0 for G <= h < 8.  Both run
// on the first 8*D/8 threads (whole waves).  Rows are padded to QS = D + 4
// floats so that the 16-byte operand reads of different heads fall in
// different LDS banks.
template <int D>
constexpr int kQS = D + 4;
struct QueryIn {
  float v[8];
  uint32_t sb;
};
template <int D>
__device__ __forceinline__ void load_query(const float* q, const uint32_t* mask, int G, int tid,
                                           QueryIn& Q) {
  constexpr int LPV = D / 8;
  const int h = tid / LPV, sub = tid % LPV;
  if (tid < kMaxG * LPV && h < G) {
    const float4* p = reinterpret_cast<const float4*>(q + h * D + 8 * sub);
    const float4 a = p[0], b = p[1];
    Q.v[0] = a.x; Q.v[1] = a.y; Q.v[2] = a.z; Q.v[3] = a.w;
    Q.v[4] = b.x; Q.v[5] = b.y; Q.v[6] = b.z; Q.v[7] = b.w;
    Q.sb = sign_byte(mask, sub);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) Q.v[k] = 0.f;
    Q.sb = 0u;
  }
}
// qn, if not null, receives ||q'_h||_1 of each row (the router's error bound).
template <int D>
__device__ __forceinline__ void rotate_query(QueryIn& Q, float mult, float* qf, int tid,
                                             float* qn = nullptr) {
  constexpr int LPV = D / 8;
  if (tid < kMaxG * LPV) {
    const int h = tid / LPV, sub = tid % LPV;
#pragma unroll
    for (int k = 0; k < 8; ++k) Q.v[k] = flip(Q.v[k], (Q.sb >> k) & 1u);
    fwht8xlanes<LPV>(Q.v, sub);
    const f32x4 a = f32x4{Q.v[0], Q.v[1], Q.v[2], Q.v[3]} * mult;
    const f32x4 b = f32x4{Q.v[4], Q.v[5], Q.v[6], Q.v[7]} * mult;
    f32x4* dst = reinterpret_cast<f32x4*>(qf + h * kQS<D> + 8 * sub);
    dst[0] = a;
    dst[1] = b;
    if (qn) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) s += fabsf(a[k]) + fabsf(b[k]);
      s = group_sum<LPV>(s);
      if (sub == 0) qn[h] = s;
    }
  }
}

// B operand of the QK products: lane (c, gq) holds head col_head(c), dims
// gq*D/4 + 8m + j for k-chunk m; hi/lo fp16 split of the fp32 rotated query.
template <int D>
__device__ void query_operands(const float* qf, int lane, half8 (&hi)[D / 32],
                               half8 (&lo)[D / 32]) {
  const int c = lane & 15, gq = lane >> 4, h = col_head(c);
  const f32x4* src = reinterpret_cast<const f32x4*>(qf + h * kQS<D> + gq * (D / 4));
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const f32x4 x0 = src[2 * m], x1 = src[2 * m + 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = (j < 4) ? x0[j] : x1[j - 4];
      const _Float16 xh = (_Float16)x;
      hi[m][j] = xh;
      lo[m][j] = (_Float16)(x - (float)xh);
    }
  }
}

// B operand of the router products: lane (c, gq) holds, for column c < 8,
// the fp16 high part of head c's rotated query and, for column 8 + h, its
// low part x - fp16(x) (dims as in query_operands; rows of absent heads are
// zero).
template <int D>
__device__ void router_operands(const float* qf, int lane, half8 (&b)[D / 32]) {
  const int c = lane & 15, gq = lane >> 4, h = c & 7;
  const bool low = c >= 8;
  const f32x4* src = reinterpret_cast<const f32x4*>(qf + h * kQS<D> + gq * (D / 4));
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const f32x4 x0 = src[2 * m], x1 = src[2 * m + 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = (j < 4) ? x0[j] : x1[j - 4];
      const _Float16 xh = (_Float16)x;
      b[m][j] = low ? (_Float16)(x - (float)xh) : xh;
    }
  }
}

// TQ-QKV: uf[h][j] = mult * sum_i S[j][i] qf[h][i] for h < G (rows of absent
// heads are zero), S the unit's D x D sketch matrix (row j = direction j).
// Each 16-lane group of a wave takes one row j at a time, D/16 coordinates
// per lane (coalesced 16-byte loads), and sums over the group by DPP.
template <int D>
__device__ void qjl_project(const float* S, const float* qf, int G, float mult, float* uf,
                            int tid, int nthreads) {
  constexpr int PL = D / 16;  // coordinates per lane
  const int l16 = tid & 15, grp = tid >> 4, ngrp = nthreads >> 4;
  for (int j = grp; j < D; j += ngrp) {
    float sv[PL];
    const f32x4* sp = reinterpret_cast<const f32x4*>(S + (size_t)j * D + PL * l16);
#pragma unroll
    for (int c = 0; c < PL / 4; ++c) {
      const f32x4 x = sp[c];
      sv[4 * c] = x[0]; sv[4 * c + 1] = x[1]; sv[4 * c + 2] = x[2]; sv[4 * c + 3] = x[3];
    }
    for (int h = 0; h < kMaxG; ++h) {  // uniform within the group
      float acc = 0.f;
      if (h < G) {
        const float* qp = qf + h * kQS<D> + PL * l16;
#pragma unroll
        for (int c = 0; c < PL; ++c) acc = fmaf(sv[c], qp[c], acc);
      }
      acc = group_sum<16>(acc);
      if (l16 == 0) uf[h * kQS<D> + j] = acc * mult;
    }
  }
}
// B operand of the sketch products: lane (c, gq), chunk m, slot 2k + h holds
// head col_head(c)'s u at coordinate gq*D/4 + 4m + k + (D/8) h (the order in
// which consume_tok takes the sketch bits).
template <int D>
__device__ void qjl_operands(const float* uf, int lane, half8 (&u)[D / 32]) {
  const int c = lane & 15, gq = lane >> 4, h = col_head(c);
  const float* src = uf + h * kQS<D> + gq * (D / 4);
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) u[m][2 * k + hh] = (_Float16)src[4 * m + k + (D / 8) * hh];
}

// ---------------------------------------------------------- online softmax ---

constexpr float kLog2e = 1.4426950408889634f;
// A logit may exceed the running reference maximum by this much (natural
// log units) before the state is rescaled: weights stay <= e^4, well inside
// fp16 even after multiplication by a value norm.
constexpr float kLazy = 4.f;

// Softmax state of one lane: reference maximum m of its column (equal on the
// 4 row groups), its share l of the denominator (its 4 rows), and the MFMA
// accumulators O of the value product.
template <int D>
struct Softmax {
  float m, mL;  // mL = m * log2(e)
  float mth;    // m + kLazy
  float l;
  f32x4 O[D / 32];
  __device__ void init(float m0) {
    m = m0;
    mL = m0 * kLog2e;
    mth = m0 + kLazy;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // p_i = exp(lg_i - m)
  __device__ __forceinline__ void weights(const float (&lg)[4], float (&p)[4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(lg[i], kLog2e, -mL));
  }
  // Fold in 4 logits of this lane (rows 4gq+i) with a lazily moved maximum:
  // the state is rescaled only when a logit exceeds the reference by more
  // than kLazy (rare once the first tiles are in).  Each lane tests its own
  // rows; only a rescale takes the maximum over the column's four lanes, so
  // the lanes of a column keep one reference.
  __device__ __forceinline__ void update(const float (&lg)[4], float (&p)[4]) {
    float mt = max3f(max3f(lg[0], lg[1], lg[2]), lg[3], lg[3]);
    if (__builtin_amdgcn_ballot_w64(mt > mth)) {  // wave-uniform branch
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = (mt > mth) ? mt : m;
      const float alpha = (m == kNegInf) ? 0.f : __expf(m - mn);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) O[t] *= alpha;
      m = mn;
      mL = mn * kLog2e;
      mth = mn + kLazy;
    }
    weights(lg, p);
  }
};

// B operand of the value products from 4 weights of this lane's column
// (h, e'): token 4gq+j, element e' of each dimension pair.
__device__ __forceinline__ half8 weight_operand(const float (&w)[4], int lane) {
  const uint32_t sh = col_elem(lane & 15) ? 16u : 0u;
  uint32_t pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)w[j]) << sh;
  return as_h8(pb[0], pb[1], pb[2], pb[3]);
}

// PV with 4-bit values: va[j] = this lane's value bits of token 4gq+j (low
// bytes first); b = weight operand.
template <int D>
__device__ __forceinline__ void pv4(const uint32_t (&va)[4], half8 b, uint32_t lane4,
                                    const uint32_t* lut4, f32x4 (&O)[D / 32]) {
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
      a[j] = lds_at(lut4, addr);
    }
    O[t] = mfma16(as_h8(a[0], a[1], a[2], a[3]), b, O[t]);
  }
}

// PV with 3-bit values (hi table only: V needs no split).  va[j]: this lane's
// value bits of token 4gq+j start at bit `sh`.
template <int D>
__device__ __forceinline__ void pv3(const uint32_t (&va)[4], uint32_t sh, half8 b, uint32_t lane4,
                                    const uint32_t* lut3, f32x4 (&O)[D / 32]) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    uint32_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = lds_at(lut3, lut3_addr(__builtin_amdgcn_ubfe(va[j], sh + 6 * t, 6), lane4));
    O[t] = mfma16(as_h8(a[0], a[1], a[2], a[3]), b, O[t]);
  }
}

// Combine the waves' states; result per head written to dst[h][D+2] as
// [m, l, O[0..D)] (dst may be LDS or global).  scratch: kWaves*kMaxG*(D+2) floats.
template <int D, int NW = kWaves>
__device__ void combine_waves(const Softmax<D>& st, int G, float* scratch, float* dst, int tid,
                              int gs = kMaxG) {
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, gq = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  constexpr int T = D / 32;
  const int h = col_head(c), e = col_elem(c);
  float* w = scratch + (wave * gs + h) * (D + 2);
  if (h < G) {
    if (gq == 0 && e == 0) {
      w[0] = st.m;
      w[1] = l;
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[2 + 2 * (T * (4 * gq + i) + t) + e] = st.O[t][i];
  }
  lds_barrier();
  for (int k = tid; k < G * (D + 2); k += (NW * 64)) {
    const int hh = k / (D + 2), e = k % (D + 2);
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, scratch[(v * gs + hh) * (D + 2)]);
    float acc = 0.f;
    if (e > 0) {
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float* s = scratch + (v * gs + hh) * (D + 2);
        const float wgt = (s[0] == kNegInf) ? 0.f : __expf(s[0] - M);
        acc += wgt * s[e];
      }
    }
    dst[k] = (e == 0) ? M : acc;
  }
  lds_barrier();
}

// ------------------------------------------------------------ top-beta ------

// Ordered uint32 key of a float: larger float <-> larger key.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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


// Top-beta (0 < beta < ng) starts from a histogram of the scores over
// [lo, hi] (any bounds of the scores) in 256 equal steps, which places the
// beta-th largest score in one bucket; select_wave then counts and ranks
// keys against bounds around that bucket, so the result is the order of the
// full sort by (key descending, index ascending).

// The threshold bucket and how many of its scores to take, from the full
// histogram; every wave computes it (no barrier needed).
__device__ __forceinline__ void hist_threshold(const int* hist, int beta, int lane, int& bt,
                                               int& need) {
  int cnt[4], sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // lane l owns buckets 255-4l .. 252-4l
    cnt[k] = hist[255 - 4 * lane - k];
    sum += cnt[k];
  }
  const int incl = wave_incl_scan(sum);
  int my_bt = 0, my_need = 0, acc = incl - sum;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (acc < beta && acc + cnt[k] >= beta) {
      my_bt = 255 - 4 * lane - k;
      my_need = beta - acc;
    }
    acc += cnt[k];
  }
  const int src = __ffsll((unsigned long long)__builtin_amdgcn_ballot_w64(my_need > 0)) - 1;
  bt = __builtin_amdgcn_readlane(my_bt, src);
  need = __builtin_amdgcn_readlane(my_need, src);
}


// Exclusive prefix sum of v over the lanes of a wave, plus the wave total.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int& total) {
  (void)lane;
  const int incl = wave_incl_scan(v);
  total = __builtin_amdgcn_readlane(incl, 63);
  return incl - v;
}

// Orders the LDS accesses of one wave around this point (the wave's LDS
// operations complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Radix select of the beta-th largest of the keys key(0 .. ng-1) by one wave: 4 passes
// of 8 bits, most significant first, histogram in LDS.  Returns that key;
// need = how many of the keys equal to it rank among the beta largest.
// 0 < beta < ng.
template <typename KeyF>
__device__ uint32_t radix_kth_f(KeyF key, int ng, int beta, int* hist, int lane, int& need_out) {
  uint32_t pre = 0u, msk = 0u;
  int need = beta;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) hist[b] = 0;
    wave_lds_sync();
    for (int g = lane; g < ng; g += 64) {
      const uint32_t k = key(g);
      if ((k & msk) == pre) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    wave_lds_sync();
    int cnt[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // lane l owns bins 255-4l .. 252-4l
      cnt[k] = hist[255 - 4 * lane - k];
      sum += cnt[k];
    }
    int total;
    const int excl = wave_excl_scan(sum, lane, total);
    int my_bin = -1, my_acc = 0;
    if (excl < need && excl + sum >= need) {
      int acc = excl;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (my_bin < 0 && acc + cnt[k] >= need) {
          my_bin = 255 - 4 * lane - k;
          my_acc = acc;
        }
        acc += cnt[k];
      }
    }
    const int src = __ffsll((unsigned long long)__builtin_amdgcn_ballot_w64(my_bin >= 0)) - 1;
    pre |= (uint32_t)__builtin_amdgcn_readlane(my_bin, src) << shift;
    msk |= 255u << shift;
    need -= __builtin_amdgcn_readlane(my_acc, src);
    wave_lds_sync();
  }
  need_out = need;
  return pre;
}
__device__ uint32_t radix_kth(const uint32_t* keys, int ng, int beta, int* hist, int lane,
                              int& need_out) {
  return radix_kth_f([&](int g) { return keys[g]; }, ng, beta, hist, lane, need_out);
}

// Top-beta of keys[0..ng) by one wave: sel[0..beta) ascending group ids.
// The radix select finds the key of the beta-th largest score and how many
// of its ties to take; an in-order pass then emits the selected ids, ties
// resolved to the lower index.  0 < beta < ng.  sel may alias keys (an id
// is written at or below the position of the keys still to be read).
__device__ void top_beta_wave(const uint32_t* keys, int ng, int beta, int* hist, int32_t* sel,
                              int lane) {
  int need;
  const uint32_t pre = radix_kth(keys, ng, beta, hist, lane, need);
  int pos = 0, eq_before = 0;
  for (int g0 = 0; g0 < ng; g0 += 64) {
    const int g = g0 + lane;
    const uint32_t k = g < ng ? keys[g] : 0u;
    const bool eq = g < ng && k == pre;
    int n_eq;
    const int eq_excl = wave_excl_scan(eq ? 1 : 0, lane, n_eq);
    const bool take = (g < ng && k > pre) || (eq && eq_before + eq_excl < need);
    int n_take;
    const int p = wave_excl_scan(take ? 1 : 0, lane, n_take);
    if (take) sel[pos + p] = g;
    pos += n_take;
    eq_before += n_eq;
  }
  wave_lds_sync();
}

// -------------------------------------------------------- summary kernel ---

struct SumArgs {
  const float* q;
  const uint8_t* l2k; const float* l2k_n; const uint8_t* l2v; const float* l2v_n;
  const uint32_t* k_signs; const float* cb3;
  float scale, bias;
  int agg, Hkv, G, ng, beta;
  int ngs;                 // groups between consecutive units of the L2 arrays
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
    return __builtin_amdgcn_ubfe(w[k], s, 6);
  } else {
    return __builtin_amdgcn_alignbit(w[k + 1], w[k], s) & 63u;
  }
}

// QK of 16 summaries.  b: router operand (column h < 8: q_hi of head h,
// column 8 + h: q_lo), so one MFMA chain forms both query parts and a row
// rotation by 8 adds them; lanes with column c < 8 return head c's logits.
// The keys enter as fp16 roundings of the stored centroids; with EXACT a
// second chain adds the centroids' low parts (lo table), which makes the
// logits fp32-accurate.  Without it they differ from the exact ones by at
// most r * ||q'||_1 * max |c - fp16(c)| (plus fp32 rounding), the bound the
// selection works with.  kw: this lane's 3D/4 key bits (summary lane&15,
// dims gq*D/4 ..) from bit 0.  The table reads go straight into the operand
// registers.
template <int D, bool EXACT>
__device__ __forceinline__ f32x4 qk3(const uint32_t (&kw)[3], const half8 (&b)[D / 32],
                                     const uint32_t* lut, const uint32_t* lutlo, uint32_t lane4) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
  uint32_t a[D / 8];
#define HSQ_FIELD_ADDR(P) a[P] = lut3_addr(field6<6 * (P)>(kw), lane4)
  HSQ_FIELD_ADDR(0); HSQ_FIELD_ADDR(1); HSQ_FIELD_ADDR(2); HSQ_FIELD_ADDR(3);
  HSQ_FIELD_ADDR(4); HSQ_FIELD_ADDR(5); HSQ_FIELD_ADDR(6); HSQ_FIELD_ADDR(7);
  if constexpr (D == 128) {
    HSQ_FIELD_ADDR(8); HSQ_FIELD_ADDR(9); HSQ_FIELD_ADDR(10); HSQ_FIELD_ADDR(11);
    HSQ_FIELD_ADDR(12); HSQ_FIELD_ADDR(13); HSQ_FIELD_ADDR(14); HSQ_FIELD_ADDR(15);
  }
#undef HSQ_FIELD_ADDR
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const half8 ak = as_h8(lds_at(lut, a[4 * m]), lds_at(lut, a[4 * m + 1]),
                           lds_at(lut, a[4 * m + 2]), lds_at(lut, a[4 * m + 3]));
    acc = mfma16(ak, b[m], acc);
    if constexpr (EXACT) {
      const half8 al = as_h8(lds_at(lutlo, a[4 * m]), lds_at(lutlo, a[4 * m + 1]),
                             lds_at(lutlo, a[4 * m + 2]), lds_at(lutlo, a[4 * m + 3]));
      accl = mfma16(al, b[m], accl);
    }
  }
  if constexpr (EXACT) acc += accl * (1.f / kLoScale);
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // row_ror:8 (a plain move, so that it fuses into the add)
    const int v = __float_as_int(acc[i]);
    r[i] = acc[i] + __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, true));
  }
  return r;
}

// Router score of group g with the stored fp32 centroids and fp32 sums (the
// selection's tie-break for groups near the beta-th score).  The 16 lanes of
// a row (sub = lane & 15) share the work, D/16 coordinates each; every lane
// of the row returns the score.  qf: rotated, scaled query rows; cb: the
// eight fp32 centroids.  exact_load issues the group's loads and
// exact_from does the arithmetic, so that several groups' loads can be in
// flight together.
template <int D>
struct ExactRaw {
  uint32_t w;  // this lane's code bits (D/16 codes from bit 0)
  float r;     // the key norm
};
template <int D>
__device__ __forceinline__ ExactRaw<D> exact_load(rsrc_t rk, rsrc_t rkn, int g, int sub) {
  constexpr int CB3 = 3 * D / 8, PER = D / 16;
  const uint32_t bit = 3u * PER * (uint32_t)sub;
  const uint32_t byte = min(bit >> 3, (uint32_t)(CB3 - 4));  // the dword stays inside the row
  ExactRaw<D> x;
  x.w = ld32(rk, (uint32_t)g * CB3 + byte);
  x.r = __uint_as_float(ld32(rkn, (uint32_t)g * 4u));
  x.w >>= bit - 8u * byte;
  return x;
}
template <int D>
__device__ __forceinline__ float exact_from(const ExactRaw<D>& x, int sub, const float* qf,
                                            const float* cb, int G, bool mean) {
  constexpr int PER = D / 16;
  float cv[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) cv[k] = cb[(x.w >> (3 * k)) & 7u];
  float best = kNegInf, sum = 0.f;
  for (int h = 0; h < G; ++h) {
    const float* qr = qf + h * kQS<D> + PER * sub;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc = __builtin_fmaf(qr[k], cv[k], acc);
    acc = group_sum<16>(acc);
    const float lg = acc * x.r;
    best = fmaxf(best, lg);
    sum += lg;
  }
  return mean ? sum * (1.f / (float)G) : best;
}
template <int D>
__device__ __forceinline__ float exact_score(rsrc_t rk, rsrc_t rkn, int g, int sub, const float* qf,
                                             const float* cb, int G, bool mean) {
  return exact_from<D>(exact_load<D>(rk, rkn, g, sub), sub, qf, cb, G, mean);
}
// exact_from for P groups at once (P passes of four): each head's query
// slice is read once for all of them.
template <int D, int P>
__device__ __forceinline__ void exact_from_p(const ExactRaw<D> (&x)[P], int sub, const float* qf,
                                             const float* cb, int G, bool mean, float (&out)[P]) {
  constexpr int PER = D / 16;
  float cv[P][PER];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int k = 0; k < PER; ++k) cv[p][k] = cb[(x[p].w >> (3 * k)) & 7u];
  float best[P], sum[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    best[p] = kNegInf;
    sum[p] = 0.f;
  }
  for (int h = 0; h < G; ++h) {
    const float* qr = qf + h * kQS<D> + PER * sub;
    float q[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) q[k] = qr[k];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc = __builtin_fmaf(q[k], cv[p][k], acc);
      acc = group_sum<16>(acc);
      const float lg = acc * x[p].r;
      best[p] = fmaxf(best[p], lg);
      sum[p] += lg;
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) out[p] = mean ? sum[p] * (1.f / (float)G) : best[p];
}

// Keys of tile t (16 summaries): this lane's raw key words (D = 128: 96 bits
// at byte 12gq of row lane&15; D = 64: 64 bits from the dword holding bit
// 48gq, aligned by key_bits) and the key norm of row 4gq + (lane & 3).
struct KeyTile {
  uint32_t kw[3];
  float kn;  // norm of row 4gq + (lane & 3) (see mul_rows)
};
template <int D>
__device__ __forceinline__ void load_keys(rsrc_t rk, rsrc_t rn, int t, int lane,
                                          KeyTile& T) {
  constexpr int CB3 = 3 * D / 8;
  const int n = lane & 15, gq = lane >> 4;
  const uint32_t row = (uint32_t)(16 * t + n) * CB3;
  if constexpr (D == 128) {
    const u32x3 w = ld96(rk, row + 12 * gq);
    T.kw[0] = w.x; T.kw[1] = w.y; T.kw[2] = w.z;
  } else {
    const u32x2 w = ld64(rk, row + 4 * ((3 * gq) >> 1));
    T.kw[0] = w.x; T.kw[1] = w.y; T.kw[2] = 0u;
  }
  T.kn = __uint_as_float(ld32(rn, (uint32_t)(16 * t + 4 * gq + (lane & 3)) * 4));
}
// This lane's key bits from the words load_keys left (the loads stay free of
// arithmetic so that no wait is forced before the tile is used).
template <int D>
__device__ __forceinline__ void key_bits(const uint32_t (&w)[3], int lane, uint32_t (&kw)[3]) {
  if constexpr (D == 128) {
    kw[0] = w[0]; kw[1] = w[1]; kw[2] = w[2];
  } else {
    const uint32_t s = ((lane >> 4) & 1) ? 16u : 0u;
    kw[0] = __builtin_amdgcn_alignbit(w[1], w[0], s);
    kw[1] = w[1] >> s;
    kw[2] = 0u;
  }
}

// Values of tile t: the dword of row 4gq+j that holds this lane's value bits
// (dims [2T*rho, 2T*rho + 2T), T = D/32; the bits start at val_shift) and the
// norm of row 4gq + (lane & 3).
struct ValTile {
  uint32_t va[4];
  float vn;  // norm of row 4gq + (lane & 3) (see mul_rows)
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
__device__ __forceinline__ void load_vals(rsrc_t rv, rsrc_t rvn, int t, int lane,
                                          ValTile& T) {
  constexpr int RB = 3 * D / 8;
  const int gq = lane >> 4;
  // the tile's part of the offsets is wave-uniform (scalar arithmetic)
  const uint32_t tv = (uint32_t)__builtin_amdgcn_readfirstlane(t * (16 * RB));
  const uint32_t tn = (uint32_t)__builtin_amdgcn_readfirstlane(t * 64);
  uint32_t base = tv + (uint32_t)(4 * gq * RB) + val_byte<D>(lane);
  // kept opaque so that the row steps j * RB become immediate offsets of
  // the loads (range-checked like the register part) instead of adds
  asm("" : "+v"(base));
#pragma unroll
  for (int j = 0; j < 4; ++j) T.va[j] = ld32(rv, base + j * RB);
  T.vn = __uint_as_float(ld32(rvn, tn + (uint32_t)(16 * gq + 4 * (lane & 3))));
}

// Byte offsets of the route body's LDS arrays after `base` (16-byte aligned):
// [logits G*ngp f32][keys u32, then the emitted selection][hist 256]
// [fetched bitmap][the threshold bucket's groups (uint2 x 64)].
struct RouteLayout {
  int logits, keys, hist, fmask, cand, end;
};
__host__ __device__ inline RouteLayout route_layout(int G, int ng, int beta, int base) {
  (void)beta;
  const int ngp = (ng + 15) & ~15;
  const int words4 = ((ngp + 31) / 32 + 3) & ~3;
  RouteLayout r;
  r.logits = base;
  r.keys = r.logits + G * ngp * 4;
  r.hist = r.keys + ((ngp + 31) & ~31) * 4;
  r.fmask = r.hist + 256 * 4;
  r.cand = r.fmask + words4 * 4;
  r.end = r.cand + 64 * 8;
  return r;
}

// LDS used by the route body.  lut3 and the tables' users are inlined, so a
// table at a fixed address folds into the reads' offsets.
struct RouteLds {
  uint32_t* lut3;   // 64 * kNC3 words
  uint32_t* lut3lo; // low parts, 64 * kNC3 words (exact router only)
  float* qf;        // rotated query rows, kMaxG * kQS<D>
  float* logits;
  uint32_t* keys;
  int* hist;
  uint32_t* fmask;
  uint2* cand;
  float* dummy;     // 64 x 4 floats: landing slot of the lanes without a head
  float* scratch;   // wave-combine scratch, kWaves * kMaxG * (D+2) floats, free
                    // once the logits are no longer needed
};
template <int D>
__device__ __forceinline__ RouteLds route_lds(char* base, const RouteLayout& r, uint32_t* lut3,
                                              float* qf, float* dummy, float* scratch) {
  RouteLds L;
  L.lut3 = lut3;
  L.lut3lo = nullptr;
  L.qf = qf;
  L.logits = reinterpret_cast<float*>(base + r.logits);
  L.keys = reinterpret_cast<uint32_t*>(base + r.keys);
  L.hist = reinterpret_cast<int*>(base + r.hist);
  L.fmask = reinterpret_cast<uint32_t*>(base + r.fmask);
  L.cand = reinterpret_cast<uint2*>(base + r.cand);
  L.dummy = dummy;
  L.scratch = scratch;
  return L;
}

// Top-beta of the unit's router keys by one wave (groups within bnd of the
// threshold are ranked by their exact scores), emitted in ascending
// order: into io.keys[0..beta) (the keys array is
// reused), io.idx, io.recoff (record offsets) and io.bits (bitmap of the
// selected groups, whole words) when those are set.  Without hsel the
// selection is io.fmask.  Returns the number of groups selected.
struct SelIo {
  uint32_t* keys;          // LDS [ng] order-preserving keys; receives the selection
  int* hist;               // LDS [256], the score histogram over [lo, hi]
  uint2* cand;             // LDS [64]
  const uint32_t* fmask;   // LDS bitmap: the selection when !hsel
  int words, ng, beta, G;
  float lo, bscale, bnd;
  bool hsel, mean;
  rsrc_t rk, rkn;          // summary key codes and norms of the unit (rescoring)
  const float* qf;         // rotated query rows
  const float* cb;         // the eight fp32 centroids
  int32_t* idx;            // out [beta] or null
  int32_t* recoff;         // LDS out [beta] or null
  uint32_t rec;            // record bytes (recoff = g * rec)
  uint32_t* bits;          // out [words] bitmap or null
};
// Key bounds [Klo, Khi) of the scores in buckets bt-1 .. bt+1 of the
// histogram over [lo, lo + 256 / bscale]; false when the histogram's range is
// degenerate.  Keys at the bounds may land one bucket off the histogram's own
// rounding; the selection counts keys against the bounds, never the
// histogram's counts, so only the bounds' order matters.
__device__ __forceinline__ bool c_bounds(int bt, float lo, float bscale, uint32_t& Klo,
                                         uint32_t& Khi) {
  const float step = 1.f / bscale;
  if (!(bscale > 0.f && __builtin_isfinite(step) && __builtin_isfinite(lo))) return false;
  const int blb = max(bt - 1, 0), bup = bt + 2;
  Klo = blb == 0 ? 0u : fkey(lo + (float)blb * step);
  Khi = bup > 255 ? 0xffffffffu : fkey(lo + (float)bup * step);
  return true;
}

template <int D, bool EXACT>
__device__ int select_wave(const SelIo& io, int lane) {
  const int sub = lane & 15, row = lane >> 4;
  const float bnd = io.bnd;
  constexpr uint32_t kMark = 0xffffffffu;  // key of a chosen group (see below)
  const int nkey = 32 * io.words;          // entries of the keys array
  // keys of the band's edges around theta (a bound that is not finite,
  // from overflowing inputs, puts every group in the band)
  auto band_keys = [&](uint32_t theta, uint32_t& khi, uint32_t& klo) {
    if constexpr (EXACT) {
      khi = klo = theta;
    } else {
      const float tf = key_float(theta);
      const float tup = tf + 2.f * bnd, tdn = tf - 2.f * bnd;
      const bool fin = __builtin_isfinite(tup) && __builtin_isfinite(tdn);
      khi = fin ? fkey(tup) : 0xffffffffu;
      klo = fin ? fkey(tdn) : 0u;
    }
  };
  // exact keys of listed groups io.cand[0..n) (into io.cand[j].y), four
  // groups per pass (16 lanes each), the loads of four passes issued
  // together; the exact router's keys are exact already
  auto rescore = [&](int n) {
    if constexpr (!EXACT) {
      constexpr int P = 4;
      for (int j0 = 0; j0 < n; j0 += 4 * P) {
        ExactRaw<D> raw[P];
        int jj[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
          jj[p] = min(j0 + 4 * p + row, n - 1);
          raw[p] = ExactRaw<D>{0u, 0.f};
          if (j0 + 4 * p < n)  // wave-uniform
            raw[p] = exact_load<D>(io.rk, io.rkn, (int)io.cand[jj[p]].x, sub);
        }
        float sc[P];
        exact_from_p<D, P>(raw, sub, io.qf, io.cb, io.G, io.mean, sc);
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (sub == 0 && j0 + 4 * p + row < n) io.cand[jj[p]].y = fkey(sc[p]);
      }
      wave_lds_sync();
    }
  };
  // rank of this lane's (key, id) among lanes [0, n): (key desc, id asc)
  auto rank_of = [&](uint2 me, int n) {
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const uint32_t og = __builtin_amdgcn_readlane(me.x, j);
      const uint32_t ok = __builtin_amdgcn_readlane(me.y, j);
      rank += (ok > me.y) || (ok == me.y && og < me.x);
    }
    return rank;
  };
  // Every path below ends in the same form: the selection is the groups
  // whose key is >= kth once the chosen groups near the threshold have had
  // their key replaced by kMark (none of them compares >= kth before).
  uint2 me = make_uint2(0u, 0u), bme = make_uint2(0u, 0u);
  uint64_t mask_a = 0u, mask_b = 0u;  // chosen lanes of me / of bme
  uint32_t kth = kMark;
  bool fast = false;
  // Fast path.  The histogram's threshold bucket bt gives key bounds
  // [Klo, Khi) around buckets bt-1 .. bt+1; one pass over the keys counts
  // the groups at or above Khi exactly and lists C, those in [Klo, Khi).
  // When the beta-th key lies in C (and C fits a wave), theta = that key is
  // found bit by bit from C's keys, and if the band [theta - 2 bnd,
  // theta + 2 bnd] lies inside [Klo, Khi), every group at or above Khi is
  // above the band and every group below Klo below it; only the band's
  // groups need their exact keys.
  if (io.hsel) {
    int bt, need_h;
    hist_threshold(io.hist, io.beta, lane, bt, need_h);
    uint32_t Klo = 0u, Khi = 0u;
    int n_hi = 0, nc = 0;
    const bool have = c_bounds(bt, io.lo, io.bscale, Klo, Khi);
    if (have) {
      for (int b0 = 0; b0 < io.ng; b0 += 2048) {  // 8 reads of 4 keys per lane
        u32x4 k4[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          k4[q] = *reinterpret_cast<const u32x4*>(io.keys + min(b0 + 256 * q + 4 * lane, nkey - 4));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int g = b0 + 256 * q + 4 * lane + e;
            const uint32_t k = k4[q][e];
            const bool in = g < io.ng;
            n_hi += __popcll(__builtin_amdgcn_ballot_w64(in && k >= Khi));
            const uint64_t inc = __builtin_amdgcn_ballot_w64(in && k >= Klo && k < Khi);
            if (inc) {  // wave-uniform
              const int p = nc + (int)__builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(inc >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)inc, 0u));
              if (((inc >> lane) & 1u) && p < 64) io.cand[p] = make_uint2((uint32_t)g, k);
              nc += __popcll(inc);
            }
          }
      }
      wave_lds_sync();
      const int need = io.beta - n_hi;
      if (need > 0 && need <= nc && nc <= 64) {
        me = lane < nc ? io.cand[lane] : make_uint2(0u, 0u);
        // theta: the largest t with at least `need` keys of C >= t
        uint32_t t = 0u;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t c = t | (1u << bit);
          if (__popcll(__builtin_amdgcn_ballot_w64(lane < nc && me.y >= c)) >= need) t = c;
        }
        uint32_t khi, klo;
        band_keys(t, khi, klo);
        fast = Klo <= klo && khi < Khi;
        if (fast) {
          mask_a = __builtin_amdgcn_ballot_w64(lane < nc && me.y > khi);
          const int need2 = need - __popcll(mask_a);
          const uint64_t bm = __builtin_amdgcn_ballot_w64(lane < nc && me.y >= klo && me.y <= khi);
          const int nb = __popcll(bm);
          const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
          // the band's groups, listed in cand and rescored
          wave_lds_sync();
          if ((bm >> lane) & 1u) io.cand[pos] = me;
          wave_lds_sync();
          rescore(nb);
          bme = lane < nb ? io.cand[lane] : make_uint2(0u, 0u);
          const int rb = rank_of(bme, nb);
          mask_b = __builtin_amdgcn_ballot_w64(lane < nb && rb < need2);
          kth = Khi;
        }
      }
    }
  }
  // General path (heavy ties, or a band reaching past C): theta by radix
  // select over all keys and the band by a scan of all keys; a band of
  // more than 64 groups rescores every group, and the radix select over
  // the exact keys emits the selection.
  bool radix = false;
  if (io.hsel && !fast) {
    int nd;
    const uint32_t theta = radix_kth(io.keys, io.ng, io.beta, io.hist, lane, nd);
    uint32_t khi_e, klo;
    band_keys(theta, khi_e, klo);
    int n_above = 0, nb = 0;
    for (int w0 = 0; w0 < io.words; w0 += 64) {
      const int w = w0 + lane, wr = min(w, io.words - 1);
      u32x4 k4[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) k4[q] = *reinterpret_cast<const u32x4*>(io.keys + 32 * wr + 4 * q);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t above = 0u, inb = 0u;
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k = k4[q][e];
          const bool in = 32 * w + 4 * q + e < io.ng;
          above |= (in && k > khi_e) ? 1u << (4 * q + e) : 0u;
          inb |= (in && k >= klo && k <= khi_e) ? 1u << (4 * q + e) : 0u;
        }
      int tot_a;
      wave_excl_scan(__popc(above), lane, tot_a);
      n_above += tot_a;
      int total;
      int pos = nb + wave_excl_scan(__popc(inb), lane, total);
      while (inb) {
        if (pos < 64) io.cand[pos] = make_uint2((uint32_t)(32 * w + __ffs(inb) - 1), 0u);
        ++pos;
        inb &= inb - 1u;
      }
      nb += total;
    }
    wave_lds_sync();
    if (nb <= 64) {
      if constexpr (EXACT) {
        if (lane < nb) io.cand[lane].y = io.keys[io.cand[lane].x];
        wave_lds_sync();
      }
      rescore(nb);
      bme = lane < nb ? io.cand[lane] : make_uint2(0u, 0u);
      const int rb = rank_of(bme, nb);
      mask_b = __builtin_amdgcn_ballot_w64(lane < nb && rb < io.beta - n_above);
      kth = khi_e == kMark ? kMark : khi_e + 1u;
    } else {
      if constexpr (!EXACT) {
        for (int g0 = 0; g0 < io.ng; g0 += 4) {
          const int g = min(g0 + row, io.ng - 1);
          const uint32_t k = fkey(exact_score<D>(io.rk, io.rkn, g, sub, io.qf, io.cb, io.G, io.mean));
          if (sub == 0 && g0 + row < io.ng) io.keys[g] = k;
        }
        wave_lds_sync();
      }
      top_beta_wave(io.keys, io.ng, io.beta, io.hist, reinterpret_cast<int32_t*>(io.keys), lane);
      radix = true;
    }
  }
  // the chosen groups near the threshold take the key kMark
  if (io.hsel && !radix) {
    if ((mask_a >> lane) & 1u) io.keys[me.x] = kMark;
    if ((mask_b >> lane) & 1u) io.keys[bme.x] = kMark;
    wave_lds_sync();
  }
  // emit the selection in ascending order (the radix select already did)
  int nsel = 0;
  if (radix) {
    nsel = io.beta;
    for (int pos = lane; pos < nsel; pos += 64) {
      const int g = (int)io.keys[pos];
      if (io.idx) io.idx[pos] = g;
      if (io.recoff) io.recoff[pos] = (int32_t)((uint32_t)g * io.rec);
      if (io.bits) atomicOr(&io.bits[g >> 5], 1u << (g & 31));
    }
  } else {
    // lane w holds word w's bits (groups 32w .. 32w+31); an id is written at
    // or below the position of the keys still to be read
    for (int w0 = 0; w0 < io.words; w0 += 64) {
      const int w = w0 + lane;
      uint32_t bits = 0u;
      if (io.hsel) {
        const int wr = min(w, io.words - 1);
        u32x4 k4[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) k4[q] = *reinterpret_cast<const u32x4*>(io.keys + 32 * wr + 4 * q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = 32 * w + 4 * q + e < io.ng;
            bits |= (in && k4[q][e] >= kth) ? 1u << (4 * q + e) : 0u;
          }
      } else {
        bits = (w < io.words) ? io.fmask[w] : 0u;
      }
      if (io.bits && w < io.words) io.bits[w] = bits;
      int total;
      int pos = nsel + wave_excl_scan(__popc(bits), lane, total);
      while (bits) {
        const int g = 32 * w + __ffs(bits) - 1;
        io.keys[pos] = (uint32_t)g;
        if (io.idx) io.idx[pos] = g;
        if (io.recoff) io.recoff[pos] = (int32_t)((uint32_t)g * io.rec);
        ++pos;
        bits &= bits - 1u;
      }
      nsel += total;
    }
  }
  wave_lds_sync();

  return nsel;
}

// Router, top-beta and summary partial of one unit (the whole work-group).
// The summary partial goes either, combined over the waves, to part_out
// ([G][D+2] (m, l, O), global memory), or, when st_out is not null, stays
// per wave in *st_out (reference maximum including the summary bias) for
// the attend phase of the same work-group to continue.
// recoff: if not null, LDS table that receives g * rec for selection slot s.
// pre(): called by every wave once its share of the stream (or the
// selection) is done, before the work-group waits for the selection; the
// caller issues the first loads of its next phase there.
template <int D, bool EXACT, typename PreF>
__device__ __forceinline__ void route_unit(const SumArgs& a, const RouteLds& L, float* part_out,
                                           Softmax<D>* st_out, int32_t* recoff, uint32_t rec,
                                           int unit, PreF pre) {
  constexpr int CB3 = 3 * D / 8;
  __shared__ float s_cb[8];
  __shared__ int s_nsel;   // size of the selection
  __shared__ float s_lo[kWaves], s_hi[kWaves];
  __shared__ float s_mh[kWaves][kMaxG];
  __shared__ float s_rn[kWaves];  // largest key norm seen by each wave
  __shared__ float s_qn[kMaxG];   // ||q'_h||_1 of each head's rotated query
  const int ngp = (a.ng + 15) & ~15;
  float* qf = L.qf;
  float* logits = L.logits;
  uint32_t* keys = L.keys;
  int* hist = L.hist;
  uint32_t* fmask = L.fmask;
  uint2* cand = L.cand;
  // the emitted selection reuses the keys once the threshold step is done
  // (the candidates may still be read by slower waves while it is written)
  int32_t* sel = reinterpret_cast<int32_t*>(keys);
  const uint32_t* lut3 = L.lut3;
  // Wave priorities fall as a work-group moves through the step (router 3,
  // values and selection 2, attend tiles 1, epilogue 0): where two
  // work-groups share a CU, the one that is behind gets the issue slots
  // first, instead of the older one by age, so both finish closer together.
  __builtin_amdgcn_s_setprio(3);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int kvh = unit % a.Hkv;
  const uint32_t lane4 = (uint32_t)(lane & 31) << 2;
  const int c = lane & 15, gq = lane >> 4;

  const rsrc_t rk = make_rsrc(a.l2k + (size_t)unit * a.ngs * CB3, (uint32_t)a.ng * CB3);
  const rsrc_t rkn = make_rsrc(a.l2k_n + (size_t)unit * a.ngs, (uint32_t)a.ng * 4);
  const rsrc_t rv = make_rsrc(a.l2v + (size_t)unit * a.ngs * CB3, (uint32_t)a.ng * CB3);
  const rsrc_t rvn = make_rsrc(a.l2v_n + (size_t)unit * a.ngs, (uint32_t)a.ng * 4);

  // global loads first: the set-up inputs, then the first two key tiles of
  // this wave, whose latency the set-up arithmetic below then overlaps
  const float cbv = (tid < 8) ? a.cb3[tid] : 0.f;
  QueryIn qin;
  load_query<D>(a.q + (size_t)unit * a.G * D, a.k_signs + kvh * (D / 32), a.G, tid, qin);
  KeyTile kt[kKeyDepth];
#pragma unroll
  for (int j = 0; j < kKeyDepth - 1; ++j)
    load_keys<D>(rk, rkn, wave + j * kWaves, lane, kt[j]);

  if (tid < 8) s_cb[tid] = cbv;
  rotate_query<D>(qin, a.scale * rsqrtf((float)D), qf, tid, s_qn);
  const int words = (ngp + 31) >> 5;
  for (int w = tid; w < words; w += kThreads) fmask[w] = 0u;
  for (int b = tid; b < 256; b += kThreads) hist[b] = 0;
  lds_barrier();
  build_lut3(L.lut3, s_cb, tid);
  if constexpr (EXACT) build_lut3_lo(L.lut3lo, s_cb, tid);
  half8 qb[D / 32];
  router_operands<D>(qf, lane, qb);
  lds_barrier();

  // (1) keys -> per-head logits in LDS (column h < 8 holds head h)
  const int n_tiles = ngp >> 4;
  // lanes that hold no head's logits store into a dummy slot (no branch)
  const bool writer = c < a.G;
  float* lw = writer ? logits + c * ngp + 4 * gq : L.dummy + 4 * lane;
  float blo = kPosInf, cmax = kNegInf, rn = 0.f;
  // rows of tile t past the last group (only the last tile has any)
  auto tail_rows = [&](int t) -> uint32_t {
    const int valid = a.ng - (16 * t + 4 * gq);
    return valid >= 4 ? 0u : (valid <= 0 ? 15u : (15u & ~((1u << valid) - 1u)));
  };
  {
    pipeline<kKeyDepth>(
        wave_iters(n_tiles, wave), kt,
        [&](int i, KeyTile& T) { load_keys<D>(rk, rkn, wave + i * kWaves, lane, T); },
        [&](int i, const KeyTile& T) {
          const int t = wave + i * kWaves;
          uint32_t kw[3];
          key_bits<D>(T.kw, lane, kw);
          f32x4 lg = mul_rows(qk3<D, EXACT>(kw, qb, lut3, L.lut3lo, lane4), T.kn);
          if constexpr (!EXACT) rn = fmaxf(rn, T.kn);
          *reinterpret_cast<f32x4*>(lw + (writer ? 16 * t : 0)) = lg;
          // a lower bound of every score (max or mean over heads of these
          // logits); the heads' maxima below bound them from above
          blo = min3f(min3f(blo, lg[0], lg[1]), lg[2], lg[3]);
          if (t == n_tiles - 1) {  // wave-uniform: rows past the last group
            const uint32_t tr = tail_rows(t);
#pragma unroll
            for (int r = 0; r < 4; ++r) lg[r] = ((tr >> r) & 1u) ? kNegInf : lg[r];
          }
          cmax = max3f(max3f(cmax, lg[0], lg[1]), lg[2], lg[3]);
        });
  }
  blo = wave_min(blo);
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
  const float whi = wave_max(writer ? cmax : kNegInf);  // this wave's largest logit
  if constexpr (!EXACT) rn = wave_max(rn);
  if (lane == 0) {
    s_lo[wave] = blo;
    s_hi[wave] = whi;
    s_rn[wave] = rn;
  }
  if (gq == 0 && writer) s_mh[wave][c] = cmax;
  // Phase 2.  (2a) All eight waves form the router scores of a share of the
  // groups (max or mean over the G heads) as order-preserving keys, with
  // their histogram over [lo, hi]; one barrier.  Then seven waves stream the
  // values of ALL summaries into their softmax partials (tiles w, w + 7,
  // ...); the fetched ones are subtracted at the end with the same weights.
  // The eighth wave meanwhile finds the threshold, settles the groups near
  // it and emits the selection.  (3) After one barrier all eight waves
  // subtract the fetched summaries, and a last barrier ends the route.
  constexpr int K = kValDepth;
  constexpr int kSel = kWaves - 1;  // the selecting wave
  const bool stream = a.want_partial && a.beta < a.ng;  // else the partial is empty
  const int nv = (stream && wave != kSel && wave < n_tiles) ? (n_tiles - wave + kSel - 1) / kSel : 0;
  // past its last tile a wave names tiles past the end (no reads)
  auto tile = [&](int i) { return wave + i * kSel + (i < nv ? 0 : n_tiles); };
  ValTile vt[K];
  if (wave != kSel) {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) load_vals<D>(rv, rvn, tile(j), lane, vt[j]);
  }
  lds_barrier();

  // (2a) scores and histogram, 4 groups per lane and pass, passes dealt to
  // the waves in turn
  const bool hsel = a.want_topk && a.beta > 0 && a.beta < a.ng;
  float lo = kPosInf, hi = kNegInf;
  for (int w = 0; w < kWaves; ++w) {
    lo = fminf(lo, s_lo[w]);
    hi = fmaxf(hi, s_hi[w]);
  }
  const float bscale = (hi > lo) ? 256.f / (hi - lo) : 0.f;
  const bool want_mean = a.agg != HSQ_AGG_MAX;
  if (a.want_topk) {
    const float inv_g = 1.f / (float)a.G;
    const int hl = a.G - 1;
    for (int g0 = 4 * lane + 256 * wave; g0 < 32 * words; g0 += 256 * kWaves) {
      // every head's row is read before the first use (one LDS round trip
      // per pass); the loop reads only the G rows of real heads
      f32x4 x[kMaxG];
#pragma unroll
      for (int h = 0; h < kMaxG; ++h)
        if (h <= hl) x[h] = *reinterpret_cast<const f32x4*>(logits + h * ngp + g0);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 vmax = x[0], vsum = x[0];
#pragma unroll
      for (int h = 1; h < kMaxG; ++h) {
        if (h <= hl) {  // wave-uniform
          vmax = f32x4{__builtin_amdgcn_fmed3f(vmax[0], x[h][0], kPosInf),
                       __builtin_amdgcn_fmed3f(vmax[1], x[h][1], kPosInf),
                       __builtin_amdgcn_fmed3f(vmax[2], x[h][2], kPosInf),
                       __builtin_amdgcn_fmed3f(vmax[3], x[h][3], kPosInf)};
          vsum += x[h];
        }
      }
      u32x4 k4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = g0 + e < a.ng;
        const float v = want_mean ? vsum[e] * inv_g : vmax[e];
        k4[e] = ok ? fkey(v) : 0u;
        // branch-free: a slot past the end adds 0 to bucket 0
        if (hsel) atomicAdd(&hist[ok ? score_bucket(k4[e], lo, bscale) : 0], ok ? 1 : 0);
      }
      if (EXACT && a.scores_out) {  // only the exact router's scores are written
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (g0 + e < a.ng)
            a.scores_out[(size_t)unit * a.ng + g0 + e] = want_mean ? vsum[e] * inv_g : vmax[e];
      }
      *reinterpret_cast<u32x4*>(keys + g0) = k4;
    }
  }
  if (wave == kSel) {
    if (a.want_topk && a.beta >= a.ng) {  // every group fetched
      for (int w = lane; w < words; w += 64) {
        const int left = a.ng - 32 * w;
        fmask[w] = left >= 32 ? 0xffffffffu : (left <= 0 ? 0u : ((1u << left) - 1u));
      }
    } else if (!a.want_topk && a.given) {  // the given selection
      for (int i = lane; i < a.beta; i += 64) {
        const int g = a.given[(size_t)unit * a.beta + i];
        if (g >= 0 && g < a.ng) atomicOr(&fmask[g >> 5], 1u << (g & 31));
      }
    }
  }
  lds_barrier();

  __builtin_amdgcn_s_setprio(2);
  // every weight exp(logit + bias - m) <= 1 with m the head's maximum logit
  const int hcol = min(col_head(c), a.G - 1);
  float m0 = kNegInf;
  for (int w = 0; w < kWaves; ++w) m0 = fmaxf(m0, s_mh[w][hcol]);
  Softmax<D> st;
  // the summary bias shifts every summary logit and the reference alike, so
  // the weights are taken without it and it is added to m at the end
  st.init(m0);
  const uint32_t vsh = val_shift<D>(lane);
  // sign = +1: add the rows' contributions; -1: subtract them
  auto consume = [&](const float (&lg)[4], const ValTile& V, float sign) {
    float p[4], w[4];
    st.weights(lg, p);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st.l += sign * p[r];
      w[r] = sign * p[r] * row_norm(V.vn, r);
    }
    pv3<D>(V.va, vsh, weight_operand(w, lane), lane4, lut3, st.O);
  };
  const float* lrow = logits + hcol * ngp + 4 * gq;

  if (wave != kSel) {
    pipeline<K>(
        nv, vt, [&](int i, ValTile& V) { load_vals<D>(rv, rvn, tile(i), lane, V); },
        [&](int i, const ValTile& V) {
          const int t = tile(i);
          const f32x4 lg4 = *reinterpret_cast<const f32x4*>(lrow + 16 * t);
          float lg[4] = {lg4[0], lg4[1], lg4[2], lg4[3]};
          if (t == n_tiles - 1) {  // wave-uniform
            const uint32_t tr = tail_rows(t);
#pragma unroll
            for (int r = 0; r < 4; ++r) lg[r] = ((tr >> r) & 1u) ? kNegInf : lg[r];
          }
          consume(lg, V, 1.f);
        });
  } else {
    // this wave gates the work-group's finish: its selection goes first
    __builtin_amdgcn_s_setprio(3);
    const int sub = lane & 15, row = lane >> 4;
    // The computed scores differ from the exact ones by at most bnd (zero
    // with the exact router): r_max * max_h ||q'_h||_1 * (max |c - fp16(c)|
    // + c_max 2^-14), the fp16 centroids plus the fp32 rounding of the MFMA
    // sums and of the query split (both far below 2^-14 of the terms).  So
    // the beta-th exact score lies within bnd of the beta-th computed one,
    // theta: groups above theta + 2 bnd are taken, groups below theta - 2 bnd
    // are not, and those between (the band) are ranked by exact scores
    // (fp32 centroids and sums), then by index.
    float bnd = 0.f;
    if constexpr (!EXACT) {
      if (hsel) {
        float rmax = 0.f, qn = 0.f;
        for (int w = 0; w < kWaves; ++w) rmax = fmaxf(rmax, s_rn[w]);
        for (int h = 0; h < a.G; ++h) qn = fmaxf(qn, s_qn[h]);
        const float cl = lane < 8 ? s_cb[lane] : 0.f;
        const float dl = wave_max(fabsf(cl - (float)(_Float16)cl));
        const float cm = wave_max(fabsf(cl));
        bnd = rmax * qn * (dl + cm * 0x1p-14f) * 1.0625f;
      }
    }
    SelIo io;
    io.keys = keys; io.hist = hist; io.cand = cand; io.fmask = fmask;
    io.words = words; io.ng = a.ng; io.beta = a.beta; io.G = a.G;
    io.lo = lo; io.bscale = bscale; io.bnd = bnd; io.hsel = hsel; io.mean = want_mean;
    io.rk = rk; io.rkn = rkn; io.qf = qf; io.cb = s_cb;
    io.idx = (a.want_topk && a.idx) ? a.idx + (size_t)unit * a.beta : nullptr;
    io.recoff = recoff; io.rec = rec; io.bits = nullptr;
    const int nsel = select_wave<D, EXACT>(io, lane);
    if (lane == 0) s_nsel = nsel;
    __builtin_amdgcn_s_setprio(2);
  }
  // the caller's first loads of its next phase, in flight across the barrier
  pre();
  if (!a.want_partial) return;
  lds_barrier();  // the selection is visible to every wave
  if (stream) {
    // (3) subtract the fetched summaries (list tiles of 16, dealt to the
    // waves in turn) with the same arithmetic as they were added; rows past
    // the list read nothing
    const int nsel = __builtin_amdgcn_readfirstlane(s_nsel);
    constexpr int RB = 3 * D / 8;
    const uint32_t vb = val_byte<D>(lane);
    const int ntl = (nsel + 15) / 16;
    const int nci = wave_iters(ntl, wave);
    struct CorrTile {
      ValTile V;
      float lg[4];
    };
    // The list rows of the wave's next tile are read while the current
    // tile's loads are issued (a tile past the list rereads the last one);
    // the logits are masked at their use, so no load waits on LDS.
    const float* lcol = logits + hcol * ngp;
    auto sel_rows = [&](int i) {
      const int j = min(wave + i * kWaves, max(ntl - 1, 0));
      return *reinterpret_cast<const u32x4*>(sel + 16 * j + 4 * gq);
    };
    u32x4 gnext = sel_rows(0);
    auto corr_load = [&](int i, CorrTile& C) {
      const u32x4 g4 = gnext;
      gnext = sel_rows(i + 1);
      const int j = wave + i * kWaves;
      uint32_t nof = kFar;  // this lane's norm row: 4gq + (lane & 3)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool in = 16 * j + 4 * gq + r < nsel;
        const uint32_t g = in ? g4[r] : 0u;
        const uint32_t far = in ? 0u : kFar;
        uint32_t vo = (g * RB + vb) | far;
        asm("" : "+v"(vo));  // one load at one address per row
        C.V.va[r] = ld32(rv, vo);
        nof = (r == (lane & 3)) ? ((g * 4u) | far) : nof;
        C.lg[r] = lcol[g];
      }
      C.V.vn = __uint_as_float(ld32(rvn, nof));
    };
    constexpr int KC = 2;
    CorrTile ct[KC];
#pragma unroll
    for (int j = 0; j < KC - 1; ++j) corr_load(j, ct[j]);
    pipeline<KC>(nci, ct, corr_load, [&](int i, const CorrTile& C) {
      const int j = wave + i * kWaves;
      float lg[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) lg[r] = (16 * j + 4 * gq + r < nsel) ? C.lg[r] : kNegInf;
      consume(lg, C.V, -1.f);
    });
  }
  lds_barrier();  // the logits are no longer needed: reuse as scratch
  st.m += a.bias;
  if (st_out) {
    st.mL = st.m * kLog2e;
    st.mth = st.m + kLazy;
    *st_out = st;
    return;
  }
  combine_waves<D>(st, a.G, L.scratch, part_out, tid);
}

// EXACT: the router adds the centroids' low parts (fp32-accurate scores,
// used when the scores are returned); else the selection's band rescoring
// keeps the selected set exact.
template <int D, bool EXACT>
__global__ __launch_bounds__(kThreads) void summary_kernel(SumArgs a) {
  // dynamic layout: [qf 8*(D+4) f32][landing slot of the phase-1 stores of
  // lanes that hold no head, 64 x 16 B][route_layout]; the rotated query is
  // read again by the selection's rescoring, so nothing else lands on it.
  // The wave-combine scratch reuses the front once the tiles are done.
  extern __shared__ __align__(16) char smem[];
  __shared__ __align__(16) uint32_t s_lut3[64 * kNC3];
  __shared__ __align__(16) uint32_t s_lut3lo[EXACT ? 64 * kNC3 : 4];
  float* qf = reinterpret_cast<float*>(smem);
  float* dummy = reinterpret_cast<float*>(smem + kMaxG * kQS<D> * 4);
  const RouteLayout r = route_layout(a.G, a.ng, a.beta, kMaxG * kQS<D> * 4 + 64 * 16);
  RouteLds L = route_lds<D>(smem, r, s_lut3, qf, dummy, qf);
  L.lut3lo = s_lut3lo;
  const int unit = blockIdx.x;
  route_unit<D, EXACT>(a, L, a.part + (size_t)unit * a.G * (D + 2), nullptr, nullptr, 0u, unit,
                       [] {});
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
  int n1s, ngs;            // rows / groups between consecutive units of L1 / L3
  const float* part;       // summary partial per unit, or null when there are none
  float* out;
  // pre-RoPE archive: fp16 rows [units][beta][N][D] of the fetched keys in the
  // rotated domain (RopeKeysJob), read in place of the key codes' table
  // lookups by the fetched tiles (null otherwise)
  const uint16_t* kdense;
  // TQ-QKV token keys: the QJL sketch bits and gamma of every L1 key
  // ([units][n1][D/8], [units][n1]) and archive key ([units][ng][N][D/8],
  // [units][ng][N]), and the sketch matrices S [Hkv][D][D] (null otherwise)
  const uint8_t* l1_sk; const float* l1_gam;
  const uint8_t* l3_sk; const float* l3_gam;
  const float* S;
};

struct TokTile {
  u32x4 kw;        // key code dwords of token row lane&15 (D=64 uses .x, .y)
  float kn;        // key norm of row 4gq + (lane & 3) (see mul_rows)
  float vn;        // value norm of row 4gq + (lane & 3)
  uint32_t va[4];  // value bits of rows 4gq+j for lane rho = lane&15
};
// A tile that also carries the fetched keys' fp16 rows (pre-RoPE archive, in
// the model's domain): the lane's D/4 coordinates of token row lane&15, the
// MFMA operands as they are (D=64 uses kd[0..1]).
struct TokTileK : TokTile {
  u32x4 kd[4];
};
// A tile of TQ-QKV keys: also the lane's D/4 sketch bits of token row
// lane&15 (D = 64: 16 bits, spread to bits 0-7 and 16-23) and the gamma of
// row 4gq + (lane & 3).
struct TokTileQ : TokTile {
  uint32_t sk;
  float gm;
};

// Per-unit buffers of the token tiles.  Tile t < n1t holds L1 rows 16t ..
// 16t+15; tile n1t + f holds the fetched archive groups of slot f (N = 16) or
// of slots 2f, 2f+1 (N = 8, rows n < 8 and n >= 8).  Archive record =
// [K codes N*CB][K norms N*4][V codes N*CB][V norms N*4].
struct TokBufs {
  rsrc_t l1k, l1kn, l1v, l1vn, l3;
  rsrc_t kd;  // the unit's fetched-key rows (pre-RoPE archive), else empty
  rsrc_t l1sk, l1gm, l3sk, l3gm;  // the unit's sketches and gammas (TQ-QKV), else empty
};

template <int D, int N>
__device__ __forceinline__ TokBufs tok_bufs(const TokArgs& a, int unit) {
  constexpr int CB = D / 2;
  const size_t o1 = (size_t)unit * a.n1s;
  const size_t rec = (size_t)N * (D + 8);
  const int recs = a.l3_staged ? a.beta : a.ng;
  TokBufs B;
  B.l1k = make_rsrc(a.l1k + o1 * CB, (uint32_t)a.n1 * CB);
  B.l1kn = make_rsrc(a.l1k_n + o1, (uint32_t)a.n1 * 4);
  B.l1v = make_rsrc(a.l1v + o1 * CB, (uint32_t)a.n1 * CB);
  B.l1vn = make_rsrc(a.l1v_n + o1, (uint32_t)a.n1 * 4);
  B.l3 = make_rsrc(a.l3 + (size_t)unit * (a.l3_staged ? a.beta : a.ngs) * rec,
                   (uint32_t)(recs * rec));
  const size_t kdu = (size_t)a.beta * N * D;  // fp16 values per unit
  B.kd = make_rsrc(a.kdense ? a.kdense + (size_t)unit * kdu : nullptr,
                   a.kdense ? (uint32_t)(kdu * 2) : 0u);
  // each sketch array on its own: a tier without entries may pass null
  const size_t n3 = (size_t)a.ng * N;  // archive keys per unit
  B.l1sk = make_rsrc(a.l1_sk ? a.l1_sk + o1 * (D / 8) : nullptr,
                     a.l1_sk ? (uint32_t)a.n1 * (D / 8) : 0u);
  B.l1gm = make_rsrc(a.l1_gam ? a.l1_gam + o1 : nullptr, a.l1_gam ? (uint32_t)a.n1 * 4 : 0u);
  B.l3sk = make_rsrc(a.l3_sk ? a.l3_sk + (size_t)unit * a.ngs * N * (D / 8) : nullptr,
                     a.l3_sk ? (uint32_t)(n3 * (D / 8)) : 0u);
  B.l3gm = make_rsrc(a.l3_gam ? a.l3_gam + (size_t)unit * a.ngs * N : nullptr,
                     a.l3_gam ? (uint32_t)(n3 * 4) : 0u);
  return B;
}

// The lane's sketch bits of a key row (D/8 bytes at row_off): coordinates
// gq*D/4 .. gq*D/4 + D/4 - 1.  D = 64: 16 bits, spread so that bits 0-7
// stay and bits 8-15 move to 16-23 (the pairs the operand builder takes).
// Bit offsets past the buffer (kFar rows) read zero.
template <int D>
__device__ __forceinline__ uint32_t sketch_bits(rsrc_t r, uint32_t row_off, int gq) {
  if constexpr (D == 128) {
    return ld32(r, row_off + 4u * (uint32_t)gq);
  } else {
    const uint32_t w = ld32(r, row_off + 4u * (uint32_t)(gq >> 1)) >> (16 * (gq & 1));
    return (w & 0xffu) | ((w & 0xff00u) << 8);
  }
}

// recoff[s]: byte offset of slot s's record in the unit's archive buffer, or
// kFar (reads zero) for a slot without a valid group; recoff[beta] = kFar.
// Loads of tile t: straight-line code for both kinds (the wave-uniform kind
// picks the buffers, per-lane selects pick the offsets).
// Loads of tile t given the record offsets bk (key rows) and br (value
// rows, norms) of its archive slot(s); an L1 tile ignores them.
// FRESH: the lane's address parts are recomputed from lane_now() (for
// kernels whose pipelines run at the register limit).
template <int D, int N, bool FRESH = false, typename TT = TokTile>
__device__ __forceinline__ void load_tok_at(const TokBufs& B, int t, int n1t, int n1, uint32_t bk,
                                            uint32_t br, int lane, TT& T, int s0 = 0) {
  constexpr int CB = D / 2;
  constexpr uint32_t KB = D / 8;  // key code bytes per lane
  if constexpr (FRESH) lane = lane_now();
  const int n = lane & 15, gq = lane >> 4;
  const int tk = (N == 16) ? n : (n & 7);            // key row within the group
  const int tr = (N == 16) ? 4 * gq : 4 * (gq & 1);  // first value row within the group
  const uint32_t vl = (D == 128) ? 4u * n : 4u * (n >> 1);  // this lane's value dword
  // Two straight-line forms with the same loads (so the waits stay exact);
  // the tile's part of the L1 offsets is wave-uniform (scalar arithmetic).
  // An archive offset built on kFar stays past the end of every buffer.
  if (t < n1t) {  // wave-uniform
    const uint32_t tc = (uint32_t)__builtin_amdgcn_readfirstlane(t * (16 * CB));
    const uint32_t tn = (uint32_t)__builtin_amdgcn_readfirstlane(t * 64);
    uint32_t vo = tc + (uint32_t)(4 * gq * CB) + vl;
    asm("" : "+v"(vo));  // the row steps j * CB become immediate offsets
    if constexpr (D == 128) {
      T.kw = ld128(B.l1k, tc + (uint32_t)(n * CB) + KB * gq);
    } else {
      const u32x2 w = ld64(B.l1k, tc + (uint32_t)(n * CB) + KB * gq);
      T.kw = u32x4{w.x, w.y, 0u, 0u};
    }
    T.kn = __uint_as_float(ld32(B.l1kn, tn + (uint32_t)(16 * gq + 4 * (lane & 3))));
    T.vn = __uint_as_float(ld32(B.l1vn, tn + (uint32_t)(16 * gq + 4 * (lane & 3))));
#pragma unroll
    for (int j = 0; j < 4; ++j) T.va[j] = ld32(B.l1v, vo + j * CB);
    if constexpr (std::is_same_v<TT, TokTileQ>) {
      T.sk = sketch_bits<D>(B.l1sk, (uint32_t)((16 * t + n) * (D / 8)), gq);
      T.gm = __uint_as_float(ld32(B.l1gm, tn + (uint32_t)(16 * gq + 4 * (lane & 3))));
    }
  } else {
    uint32_t vo = br + (uint32_t)(N * (CB + 4) + tr * CB) + vl;
    asm("" : "+v"(vo));
    if constexpr (D == 128) {
      T.kw = ld128(B.l3, bk + (uint32_t)(tk * CB) + KB * gq);
    } else {
      const u32x2 w = ld64(B.l3, bk + (uint32_t)(tk * CB) + KB * gq);
      T.kw = u32x4{w.x, w.y, 0u, 0u};
    }
    T.kn = __uint_as_float(ld32(B.l3, br + (uint32_t)(N * CB + 4 * (tr + (lane & 3)))));
    T.vn = __uint_as_float(ld32(B.l3, br + (uint32_t)(N * (2 * CB + 4) + 4 * (tr + (lane & 3)))));
#pragma unroll
    for (int j = 0; j < 4; ++j) T.va[j] = ld32(B.l3, vo + j * CB);
    if constexpr (std::is_same_v<TT, TokTileK>) {
      // row slot * N + tk of the dense keys; a slot past beta reads zeros
      const int slot = s0 + ((N == 16) ? 0 : (n >> 3));
      const uint32_t ko = (uint32_t)((slot * N + tk) * (2 * D)) + (uint32_t)(gq * (D / 2));
#pragma unroll
      for (int m = 0; m < D / 32; ++m) T.kd[m] = ld128(B.kd, ko + 16 * m);
    }
    if constexpr (std::is_same_v<TT, TokTileQ>) {
      // the group of a record offset (a constant divisor); kFar gives a
      // group past every buffer, which reads zero
      constexpr uint32_t REC = (uint32_t)(N * (D + 8));
      const uint32_t gk = bk / REC, gr = br / REC;
      T.sk = sketch_bits<D>(B.l3sk, (gk * N + (uint32_t)tk) * (D / 8), gq);
      T.gm = __uint_as_float(ld32(B.l3gm, 4u * (gr * N + (uint32_t)(tr + (lane & 3)))));
    }
  }
}
// First archive slot of tile t (wave-uniform; 0 for L1 tiles, whose loads
// ignore the record offsets).
template <int N>
__device__ __forceinline__ int tile_slot(int t, int n1t) {
  return max(t - n1t, 0) * (N == 16 ? 1 : 2);
}
// Loads of tile t, the record offsets read from recoff (which covers every
// slot a tile of the pipeline can name, see tok_slots).
template <int D, int N, bool FRESH = false, typename TT = TokTile>
__device__ __forceinline__ void load_tok(const TokBufs& B, const int32_t* recoff, int t, int n1t,
                                         int n1, int lane, TT& T) {
  if constexpr (FRESH) lane = lane_now();
  const int n = lane & 15, gq = lane >> 4;
  const int xk = (N == 16) ? 0 : (n >> 3), xr = (N == 16) ? 0 : (gq >> 1);
  const int s0 = tile_slot<N>(t, n1t);
  const int32_t* rs = recoff + s0;
  const uint32_t bk = (uint32_t)rs[xk];
  const uint32_t br = (uint32_t)rs[xr];
  load_tok_at<D, N, FRESH, TT>(B, t, n1t, n1, bk, br, lane, T, s0);
}
// Entries of the record-offset table: every slot of the fetched tiles and of
// the tiles the pipeline loads past the last one (they read kFar).  A wave's
// loads run at most 2K-2 of its tiles (8 tile indices apart) past its last.
template <int N, int NW = kWaves, int TD = kTokDepth>
__host__ __device__ constexpr int tok_slots(int beta) {
  return (N == 16 ? 1 : 2) * ((N == 16 ? beta : (beta + 1) / 2) + 2 * NW * TD);
}

// Rows of tile t that hold no token: lg = -inf.  Only the ragged last L1
// tile and archive tiles with an empty slot have any (wave-uniform test by
// the caller).
template <int N>
__device__ __forceinline__ void mask_rows(float (&lg)[4], int t, int n1t, int n1, int beta,
                                          const int32_t* recoff, int lane) {
  const int gq = lane >> 4;
  uint32_t ok;
  if (t < n1t) {
    const int valid = n1 - (16 * t + 4 * gq);
    ok = valid >= 4 ? 15u : (valid <= 0 ? 0u : ((1u << valid) - 1u));
  } else {
    const int s = tile_slot<N>(t, n1t) + ((N == 16) ? 0 : (gq >> 1));
    ok = (s < beta && recoff[s] != (int32_t)kFar) ? 15u : 0u;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) lg[i] = ((ok >> i) & 1u) ? lg[i] : kNegInf;
}

// SPLITQ: qh is the router operand (fp16 high parts of the query in columns
// c < 8, low parts in c + 8), so one row rotation completes fp32-accurate
// query products in every column.
template <int D, bool SPLITQ = false, typename MaskF, typename TT = TokTile>
__device__ __forceinline__ void consume_tok(const TT& T, bool masked, MaskF mask,
                                            const half8 (&qh)[D / 32], const uint32_t* lut4,
                                            int lane, uint32_t lane4, Softmax<D>& st,
                                            bool dense = false, const half8* uh = nullptr) {
  // two accumulators so that consecutive MFMAs do not wait on each other
  f32x4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  if constexpr (std::is_same_v<TT, TokTileK>) {
    if (dense) {  // wave-uniform: a fetched tile of a pre-RoPE archive
      // model-domain rows against the unrotated query (uh: its fp16
      // operands in LDS)
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
        acc2[m & 1] = mfma16(__builtin_bit_cast(half8, T.kd[m]), uh[m], acc2[m & 1]);
    }
  }
  if (!(std::is_same_v<TT, TokTileK> && dense)) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const uint32_t w = T.kw[m];
      const half8 av = as_h8(lds_at(lut4, lut4_addr<0>(w, lane4)), lds_at(lut4, lut4_addr<1>(w, lane4)),
                             lds_at(lut4, lut4_addr<2>(w, lane4)), lds_at(lut4, lut4_addr<3>(w, lane4)));
      acc2[m & 1] = mfma16(av, qh[m], acc2[m & 1]);
    }
  }
  f32x4 acc = acc2[0] + acc2[1];
  if constexpr (SPLITQ) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = __float_as_int(acc[i]);
      acc[i] += __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, true));
    }
  }
  float lg[4], p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lg[i] = acc[i] * row_norm(T.kn, i);
  if constexpr (std::is_same_v<TT, TokTileQ>) {
    // the QJL estimate of the residual's share: <(1 - 2 bits), u> on MFMA
    // with the +-1 operands built from the sketch bits (slot 2k + h of chunk
    // m takes bit 4m + k + (D/8) h: a shift puts both at the fp16 sign bits)
    // and u = scale sqrt(pi/2)/D S R q in the same coordinate order, times
    // gamma of the row
    f32x4 aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = ((T.sk << (15 - 4 * m - k)) & 0x80008000u) | 0x3c003c00u;
      aq = mfma16(as_h8(w[0], w[1], w[2], w[3]), uh[m], aq);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = fmaf(aq[i], row_norm(T.gm, i), lg[i]);
  }
  if (masked) mask(lg);  // wave-uniform
  st.update(lg, p);
  float w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.l += p[i];
    w[i] = p[i] * row_norm(T.vn, i);
  }
  uint32_t va[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) va[j] = (D == 128) ? T.va[j] : (T.va[j] >> (16 * (lane & 1)));
  pv4<D>(va, weight_operand(w, lane), lane4, lut4, st.O);
}

// LDS used by the attend body.  lut4 is inlined as a fixed address.
struct AttendLds {
  uint32_t* lut4;   // 256 * kNC4 words; the combine scratch once the tiles are done
  float* qf;        // rotated query rows, kMaxG * kQS<D>
  float* part;      // summary partial [G][D+2]
  int32_t* recoff;  // record offset per slot, tok_slots(beta) entries
  float* cb;        // 16 centroids of the 4-bit codebook
  uint32_t* vsb;    // V sign byte per (head, lane of the inverse rotation)
  float* uf;        // TQ-QKV: scale sqrt(pi/2)/D S R q per head, kMaxG * kQS<D>
  _Float16* qm;     // pre-RoPE: scale * q per head, unrotated, fp16 [kMaxG][D]
};

// Pre-RoPE: scale * q of the lane's coordinates into L.qm (fp16), from the
// unrotated query values load_query brought (before rotate_query).
template <int D>
__device__ __forceinline__ void stage_query_model(const QueryIn& Q, float scale, _Float16* qm,
                                                  int tid) {
  constexpr int LPV = D / 8;
  if (tid < kMaxG * LPV) {
    const int h = tid / LPV, sub = tid % LPV;
    half8 x;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (_Float16)(Q.v[k] * scale);
    *reinterpret_cast<half8*>(qm + h * D + 8 * sub) = x;
  }
}

// L1 + fetched-token attention of one unit, merged with the summary partial,
// inverse V rotation, output.  On entry every array of L except the table
// is filled and visible to all waves, and the table is free; tt[j] holds the
// loads of this wave's tile wave + 8j already when l1_issued and that tile is
// an L1 tile.  bad_flag (read after the first barrier here), if not null:
// nonzero when some slot of recoff names no record.  st_in, if not null:
// this wave's softmax state of the summary partial, which the token tiles
// continue (L.part is then not used); else the waves' states start empty
// and the combined result is merged with L.part.
template <int D, int N, typename TT = TokTile, int TD = kTokDepth>
__device__ __forceinline__ void attend_unit(const TokArgs& a, const AttendLds& L,
                                            TT (&tt)[TD], bool l1_issued,
                                            const int* bad_flag, const Softmax<D>* st_in,
                                            int unit, int tile0 = 0, int tstride = 1,
                                            float* part_out = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const uint32_t lane4 = (uint32_t)lane << 2;
  const uint32_t* lut4 = L.lut4;
  const TokBufs B = tok_bufs<D, N>(a, unit);
  const int n1t = (a.n1 + 15) / 16;
  const int nft = (N == 16) ? a.beta : (a.beta + 1) / 2;
  const int total = n1t + nft;
  constexpr int LPV = D / 8;
  __builtin_amdgcn_s_setprio(1);  // see route_unit

  // The tiles of this call: tile0, tile0 + tstride, ... below total (all of
  // them by default); wave w takes the w-th, (w+8)-th, ... of those.  Past
  // its last tile a wave names tiles just past total, whose record slots
  // read as zero.
  const int n_ck = tile0 < total ? (total - tile0 + tstride - 1) / tstride : 0;
  const int iters = wave_iters(n_ck, wave);
  auto tile_of = [&](int i) {
    return i < iters ? tile0 + tstride * (wave + i * kWaves) : total + wave + kWaves * (i - iters);
  };
  // this wave's first tiles not issued yet, loading while the table is built
#pragma unroll
  for (int j = 0; j < TD - 1; ++j)
    if (!(l1_issued && wave + j * kWaves < n1t))  // wave-uniform
      load_tok<D, N, false, TT>(B, L.recoff, tile_of(j), n1t, a.n1, lane, tt[j]);
  build_lut4(L.lut4, L.cb, tid);
  half8 qh[D / 32], ql[D / 32];
  query_operands<D>(L.qf, lane, qh, ql);
  constexpr bool QJL = std::is_same_v<TT, TokTileQ>;
  if constexpr (QJL)
    qjl_project<D>(a.S + (size_t)(unit % a.Hkv) * D * D, L.qf, a.G, 1.2533141373155003f / D, L.uf,
                   tid, kThreads);
  lds_barrier();
  half8 uh[QJL ? D / 32 : 1];
  if constexpr (QJL) qjl_operands<D>(L.uf, lane, uh);
  // pre-RoPE: the B operands of the dense rows are read from LDS per tile
  const half8* uq = uh;
  if constexpr (std::is_same_v<TT, TokTileK>)
    uq = reinterpret_cast<const half8*>(L.qm + col_head(lane & 15) * D + (lane >> 4) * (D / 4));

  Softmax<D> st;
  if (st_in)
    st = *st_in;
  else
    st.init(kNegInf);
  {
    // tiles with rows that hold no token: the ragged last L1 tile, the last
    // archive tile when its second slot is empty, every archive tile when
    // some slot names no record
    const bool any_bad = bad_flag && __builtin_amdgcn_readfirstlane(*bad_flag) != 0;
    const int ragged = (a.n1 & 15) ? n1t - 1 : -1;
    const int half = (N == 8 && (a.beta & 1)) ? total - 1 : -1;
    pipeline<TD>(
        iters, tt,
        [&](int i, TT& T) {
          // the dense-key tiles run at the register limit: lane parts afresh
          load_tok<D, N, std::is_same_v<TT, TokTileK>, TT>(B, L.recoff, tile_of(i), n1t, a.n1,
                                                          lane, T);
        },
        [&](int i, const TT& T) {
          const int t = tile_of(i);
          const bool masked = t == ragged || t == half || (any_bad && t >= n1t);
          consume_tok<D>(
              T, masked,
              [&](float (&lg)[4]) { mask_rows<N>(lg, t, n1t, a.n1, a.beta, L.recoff, lane); },
              qh, lut4, lane, lane4, st, t >= n1t, uq);
        });
  }
  lds_barrier();  // the table is no longer needed: reuse as scratch
  __builtin_amdgcn_s_setprio(0);
  float* scratch = reinterpret_cast<float*>(L.lut4);
  if (part_out) {  // this call's partial, combined over the waves
    combine_waves<D>(st, a.G, scratch, part_out, tid);
    return;
  }
  float* mine = scratch + kWaves * kMaxG * (D + 2);  // [G][D+2] this unit's token partial
  combine_waves<D>(st, a.G, scratch, mine, tid);

  // merge with the summary partial, normalise
  float* o = mine + kMaxG * (D + 2);  // [G][D]
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int k = tid + r * kThreads, h = k / D, e = k % D;
    if (k >= a.G * D) break;
    const float* mp = mine + h * (D + 2);
    const float m1 = mp[0], l1 = mp[1], v1 = mp[2 + e];
    float m2 = kNegInf, l2 = 0.f, v2 = 0.f;
    if (L.part) {
      const float* pp = L.part + h * (D + 2);
      m2 = pp[0];
      l2 = pp[1];
      v2 = pp[2 + e];
    }
    const float M = fmaxf(m1, m2);
    const float w1 = (m1 == kNegInf) ? 0.f : __expf(m1 - M);
    const float w2 = (m2 == kNegInf) ? 0.f : __expf(m2 - M);
    const float Lsum = w1 * l1 + w2 * l2;
    o[k] = (Lsum > 0.f) ? (w1 * v1 + w2 * v2) / Lsum : 0.f;
  }
  lds_barrier();
  // inverse V rotation: out = D H o / sqrt(D)
  if (tid < kMaxG * LPV) {
    const int h = tid / LPV, sub = tid % LPV;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (h < a.G) ? o[h * D + 8 * sub + k] : 0.f;
    fwht8xlanes<LPV>(v, sub);
    if (h < a.G) {
      const uint32_t sb = L.vsb[tid];
      const float sc = rsqrtf((float)D);
      float* dst = a.out + ((size_t)unit * a.G + h) * D + 8 * sub;
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = flip(v[k] * sc, (sb >> k) & 1u);
    }
  }
}

// at most 128 VGPRs so that two work-groups (the LDS limit) fit on a CU.
// TT = TokTileK: the fetched tiles multiply dense fp16 key rows (a.kdense)
// instead of looking their codes up.  TT = TokTileQ: every tile also forms
// the QJL correction of its keys (a.l1_sk ... a.S).  Both run the pipeline
// one tile shallower to make room for their registers.
template <int D, int N, typename TT = TokTile>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void token_kernel(TokArgs a) {
  constexpr int TD = std::is_same_v<TT, TokTile> ? kTokDepth : kTokDepth - 1;
  extern __shared__ __align__(16) char smem[];
  __shared__ __align__(16) uint32_t s_lut4[256 * kNC4];
  __shared__ float s_cb[16];
  __shared__ uint32_t s_vsb[kMaxG * (D / 8)];
  __shared__ int s_bad;  // some slot names no record
  // dynamic layout: [qf 8*(D+4) f32][summary partial 8*(D+2) f32]
  //   [recoff tok_slots(beta)][TQ-QKV: uf 8*(D+4) f32 | pre-RoPE: qm 8*D f16]
  AttendLds L;
  L.lut4 = s_lut4;
  L.qf = reinterpret_cast<float*>(smem);
  L.part = L.qf + kMaxG * kQS<D>;
  L.recoff = reinterpret_cast<int32_t*>(L.part + kMaxG * (D + 2));
  L.cb = s_cb;
  L.vsb = s_vsb;
  L.uf = reinterpret_cast<float*>(L.recoff + ((tok_slots<N>(a.beta) + 3) & ~3));
  L.qm = reinterpret_cast<_Float16*>(L.uf);

  const int tid = threadIdx.x, wave = wave_id();
  const int unit = blockIdx.x;
  const int kvh = unit % a.Hkv;
  const int n1t = (a.n1 + 15) / 16;
  const size_t rec = (size_t)N * (D + 8);
  constexpr int LPV = D / 8;

  // global loads first: this wave's first L1 tiles (they need no record
  // offsets), the set-up inputs and the summary partial merged at the end
  const TokBufs B = tok_bufs<D, N>(a, unit);
  TT tt[TD];
#pragma unroll
  for (int j = 0; j < TD - 1; ++j)
    if (wave + j * kWaves < n1t)  // wave-uniform
      load_tok_at<D, N, false, TT>(B, wave + j * kWaves, n1t, a.n1, kFar, kFar, tid & 63, tt[j]);
  const float cbv = (tid < 16) ? a.cb4[tid] : 0.f;
  QueryIn qin;
  load_query<D>(a.q + (size_t)unit * a.G * D, a.k_signs + kvh * (D / 32), a.G, tid, qin);
  const uint32_t vsb = (tid < kMaxG * LPV) ? sign_byte(a.v_signs + kvh * (D / 32), tid % LPV) : 0u;
  const float* ps = a.part ? a.part + (size_t)unit * a.G * (D + 2) : nullptr;
  const int np = a.G * (D + 2);
  float pv[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int k = tid + r * kThreads;
    pv[r] = (k < np) ? (ps ? ps[k] : ((k % (D + 2)) == 0 ? kNegInf : 0.f)) : 0.f;
  }
  bool bad = false;
  for (int s = tid; s < tok_slots<N>(a.beta); s += kThreads) {
    int g = -1;
    if (s < a.beta) g = a.l3_staged ? s : a.idx[(size_t)unit * a.beta + s];
    const int lim = a.l3_staged ? a.beta : a.ng;
    const bool ok = g >= 0 && g < lim;
    bad |= s < a.beta && !ok;
    L.recoff[s] = ok ? (int32_t)((uint32_t)g * (uint32_t)rec) : (int32_t)kFar;
  }
  if (tid == 0) s_bad = 0;
  if (tid < 16) s_cb[tid] = cbv;
  if (tid < kMaxG * LPV) s_vsb[tid] = vsb;
#pragma unroll
  for (int r = 0; r < 3; ++r)
    if (tid + r * kThreads < np) L.part[tid + r * kThreads] = pv[r];
  if constexpr (std::is_same_v<TT, TokTileK>) stage_query_model<D>(qin, a.scale, L.qm, tid);
  rotate_query<D>(qin, a.scale * rsqrtf((float)D), L.qf, tid);
  lds_barrier();
  if (bad) s_bad = 1;  // read after the next barrier
  attend_unit<D, N, TT, TD>(a, L, tt, true, &s_bad, nullptr, unit);
}

// ------------------------------------------------------- one-launch step ---
//
// The whole decode step on one work-group per unit (archive in device-visible
// memory, 0 < n_groups <= kFusedMaxGroups).
//   (1) One stream over the summaries.  A tile brings the keys and values of
//       16 summaries; the three-term router (fp16 centroid parts and query
//       parts, fp32 sums) forms fp32-accurate per-head logits.  Their maximum
//       (or mean) over the heads is the router score, kept in LDS; the same
//       logits weight the values in each wave's online softmax.  Nothing else
//       of a tile outlives it.
//   (2) Top-beta over the scores by all eight waves: a 256-bucket histogram
//       over the scores' range, the groups above the threshold bucket taken,
//       those inside it ranked exactly by (score descending, index
//       ascending); then the selection in ascending order as record offsets.
//       The first L1 token tiles load meanwhile.
//   (3) The fetched groups' summaries are streamed again, 16 per tile, and
//       subtracted with the same logits; the L1 tiles and the fetched tokens
//       continue the same softmax states.
//   (4) The waves' states combine; inverse V rotation; output.
//
// LDS: one static 64 KB region of 256 blocks of 256 bytes.  The low half of
// block e holds entry e of the 4-bit table (a code byte -> fp16 centroid
// pair) in 32 copies, so lane l reads copy l % 32 at (e << 8) | (l % 32) << 2,
// an address one v_perm builds from the code dword.  The high halves hold,
// again in 32 copies at (f << 8) | 128 | (l % 32) << 2, the 3-bit table
// (blocks 0..63, 6-bit field f), its low parts (blocks 64..127, one
// immediate offset away, so a field's two reads share an address) and the
// router scores (blocks 128..191, 32 per block).  Each 32-lane half of a wave
// then reads 32 different banks from any table.  Once the tiles are done the
// region is the wave-combine scratch.
constexpr int kTabBytes = 256 * 256;
constexpr uint32_t kHiHalf = 128u;
constexpr uint32_t kLoOff = 64u * 256u;  // low-part table, from the 3-bit table
constexpr int kScoreBlock = 128;
constexpr int kFusedMaxGroups = 64 * 32;
constexpr int kCandCap = 256;  // threshold-bucket groups ranked in parallel
// Waves per work-group and the pipeline depths (tiles per wave: SD in the
// summary stream, TD in the token pipeline) that its register budget allows:
// two work-groups share a CU (the LDS limit), so eight waves leave each 128
// registers per lane (WPE waves per SIMD).  Measured on the 16K-context,
// 40/8-head layer: four or five tiles deep were no faster, and four waves
// with 200 registers each streamed slower (fewer waves to hide latencies).
template <int NW> struct FusedCfg;
template <> struct FusedCfg<8> { static constexpr int SD = 3, TD = 3, WPE = 4; };
// 16 waves, one work-group per CU: layers of at most 256 units
template <> struct FusedCfg<16> { static constexpr int SD = 3, TD = 3, WPE = 4; };
constexpr int kFusedWaves = 8;
constexpr int kFusedWavesFew = 16;
constexpr int kFewUnits = 256;
constexpr int kFewGroups = 1024;
static_assert((8 + 1) * kMaxG * (128 + 2) * 4 + kMaxG * 128 * 4 <= kTabBytes,
              "the epilogue's scratch must fit in the table region");

// Both tables: the 4-bit one into the low halves (thread t writes 16-byte
// chunks t, t + 512, t + 1024, t + 1536 of entries t/8 + 64k, eight chunks
// per entry), the 3-bit one into the high halves of blocks 0..63 (chunk t)
// and its low parts into those of blocks 64..127 (chunk t + 512).  A
// thread's codebook values come straight from global memory (the loads are
// issued with the kernel's first loads), so no barrier precedes the build.
struct TabIn {
  float lo4, hi4[4];  // cb4[(t/8) % 16], cb4[t/128 + 4k]
  float c0, c1;       // cb3[(t/8) % 8], cb3[(t/64) % 8]
};
__device__ __forceinline__ TabIn load_tab_in(const float* cb4, const float* cb3, int tid) {
  TabIn in;
  in.lo4 = cb4[(tid >> 3) & 15];
#pragma unroll
  for (int k = 0; k < 4; ++k) in.hi4[k] = cb4[(tid >> 7) + 4 * k];
  in.c0 = cb3[(tid >> 3) & 7];
  in.c1 = cb3[(tid >> 6) & 7];
  return in;
}
__device__ void build_tables(uint32_t* tab, const TabIn& in, int tid) {
  u32x4* dst = reinterpret_cast<u32x4*>(tab);
  const _Float16 lo = (_Float16)in.lo4;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tid + 512 * k, e = c >> 3;  // e = t/8 + 64k: e % 16 = t/8 % 16, e / 16 = t/128 + 4k
    const uint32_t v = h2u(lo, (_Float16)in.hi4[k]);
    dst[16 * e + (c & 7)] = u32x4{v, v, v, v};
  }
  const _Float16 h0 = (_Float16)in.c0, h1 = (_Float16)in.c1;
  const int b = tid >> 3;  // f = b: cb3[f % 8], cb3[f / 8]
  const uint32_t vh = h2u(h0, h1);
  const uint32_t vl = h2u((_Float16)((in.c0 - (float)h0) * kLoScale),
                          (_Float16)((in.c1 - (float)h1) * kLoScale));
  dst[16 * b + 8 + (tid & 7)] = u32x4{vh, vh, vh, vh};
  dst[16 * (b + 64) + 8 + (tid & 7)] = u32x4{vl, vl, vl, vl};
}
// LDS byte address of router score g (scores of 4-aligned g .. g+3 are
// contiguous).
__device__ __forceinline__ uint32_t score_addr(int g) {
  return ((uint32_t)(kScoreBlock + (g >> 5)) << 8) | kHiHalf | ((uint32_t)(g & 31) << 2);
}
__device__ __forceinline__ f32x4 scores4(const uint32_t* tab, int g) {
  return *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(tab) + score_addr(g));
}

// B operand of the one-launch router: column c < 8 holds the fp16 high part
// of head c's rotated query, column 8 + c its low part.  Columns of absent
// heads copy head 0 for the maximum (it does not change a maximum) and stay
// zero for the mean (they add nothing to a sum).
template <int D>
__device__ void router_operands_pad(const float* qf, int lane, int G, bool mean,
                                    half8 (&b)[D / 32]) {
  const int c = lane & 15, gq = lane >> 4, hc = col_head(c);
  const int h = (hc >= G && !mean) ? 0 : hc;
  const bool low = c >= 8;
  const f32x4* src = reinterpret_cast<const f32x4*>(qf + h * kQS<D> + gq * (D / 4));
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const f32x4 x0 = src[2 * m], x1 = src[2 * m + 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = (j < 4) ? x0[j] : x1[j - 4];
      const _Float16 xh = (_Float16)x;
      b[m][j] = low ? (_Float16)(x - (float)xh) : xh;
    }
  }
}

// Per-head logits of 16 summaries, fp32-accurate: the fp16 centroid parts
// (hi, and lo scaled by kLoScale) against both query parts.  Lane (c, gq)
// returns head col_head(c)'s scaled logits of rows 4gq .. 4gq+3 before the
// key norm.  kw: this lane's 3D/4 key bits from bit 0.
template <int D>
__device__ __forceinline__ f32x4 qk3_exact(const uint32_t (&kw)[3], const half8 (&b)[D / 32],
                                           const uint32_t* tabh, uint32_t lane4) {
  uint32_t a[D / 8];
#define HSQ_FIELD_ADDR(P) a[P] = (field6<6 * (P)>(kw) << 8) | lane4
  HSQ_FIELD_ADDR(0); HSQ_FIELD_ADDR(1); HSQ_FIELD_ADDR(2); HSQ_FIELD_ADDR(3);
  HSQ_FIELD_ADDR(4); HSQ_FIELD_ADDR(5); HSQ_FIELD_ADDR(6); HSQ_FIELD_ADDR(7);
  if constexpr (D == 128) {
    HSQ_FIELD_ADDR(8); HSQ_FIELD_ADDR(9); HSQ_FIELD_ADDR(10); HSQ_FIELD_ADDR(11);
    HSQ_FIELD_ADDR(12); HSQ_FIELD_ADDR(13); HSQ_FIELD_ADDR(14); HSQ_FIELD_ADDR(15);
  }
#undef HSQ_FIELD_ADDR
  const uint32_t* lo = tabh + kLoOff / 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const half8 ak = as_h8(lds_at(tabh, a[4 * m]), lds_at(tabh, a[4 * m + 1]),
                           lds_at(tabh, a[4 * m + 2]), lds_at(tabh, a[4 * m + 3]));
    // kept apart from the high parts' reads: merged into two-address reads
    // they would land interleaved and need moves into the operand registers
    asm volatile("" ::: "memory");
    const half8 al = as_h8(lds_at(lo, a[4 * m]), lds_at(lo, a[4 * m + 1]),
                           lds_at(lo, a[4 * m + 2]), lds_at(lo, a[4 * m + 3]));
    acc = mfma16(ak, b[m], acc);
    accl = mfma16(al, b[m], accl);
  }
  acc += accl * (1.f / kLoScale);
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // row_ror:8 adds the query parts (columns c and c + 8)
    const int v = __float_as_int(acc[i]);
    r[i] = acc[i] + __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, true));
  }
  return r;
}

// PV with 3-bit values from the one-launch step's table (see pv3).
template <int D>
__device__ __forceinline__ void pv3_tab(const uint32_t (&va)[4], uint32_t sh, half8 b,
                                        uint32_t lane4, const uint32_t* tabh, f32x4 (&O)[D / 32]) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    uint32_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = lds_at(tabh, (__builtin_amdgcn_ubfe(va[j], sh + 6 * t, 6) << 8) | lane4);
    O[t] = mfma16(as_h8(a[0], a[1], a[2], a[3]), b, O[t]);
  }
}

// Router score of this lane's four rows: the maximum (or the sum) over the
// 16 columns of its row group; columns c and c + 8 hold the same head and
// absent heads repeat head 0 (maximum) or are zero (sum), so three row steps
// cover every head: quad_perm 1,0,3,2 and 2,3,0,1, then row_ror:4.  The
// maximum is one v_max_f32 with a DPP operand per step (fmaxf would first
// quiet both operands); the s_nop gives the DPP read of a just-written
// register its two wait states.
__device__ __forceinline__ float max_dpp_q1(float x) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float max_dpp_q2(float x) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float max_dpp_r4(float x) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf"
      : "=v"(r) : "v"(x));
  return r;
}
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <bool MEAN>
__device__ __forceinline__ f32x4 row_agg(f32x4 x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (MEAN)
      x[i] = add_dpp<0x124>(add_dpp<0x4e>(add_dpp<0xb1>(x[i])));
    else
      x[i] = max_dpp_r4(max_dpp_q2(max_dpp_q1(x[i])));
  }
  return x;
}

// Summary tile: the keys and values of 16 summaries.
struct SumTile {
  KeyTile k;
  ValTile v;
};
// Summary tile of 16 listed groups (list[16j .. 16j + 15], n entries in all;
// rows past the list read zero).
template <int D>
__device__ __forceinline__ void load_sum_list(rsrc_t rk, rsrc_t rkn, rsrc_t rv, rsrc_t rvn,
                                              const int32_t* list, int n, int j, int lane,
                                              SumTile& T) {
  constexpr int CB3 = 3 * D / 8;
  const int r = lane & 15, gq = lane >> 4;
  const int ik = 16 * j + r;
  const uint32_t gk = ik < n ? (uint32_t)list[ik] : 0u;
  const uint32_t fk = ik < n ? 0u : kFar;
  uint32_t ko = (gk * CB3 + (D == 128 ? 12u * gq : 4u * ((3u * gq) >> 1))) | fk;
  asm("" : "+v"(ko));
  if constexpr (D == 128) {
    const u32x3 w = ld96(rk, ko);
    T.k.kw[0] = w.x; T.k.kw[1] = w.y; T.k.kw[2] = w.z;
  } else {
    const u32x2 w = ld64(rk, ko);
    T.k.kw[0] = w.x; T.k.kw[1] = w.y; T.k.kw[2] = 0u;
  }
  const uint32_t vb = val_byte<D>(lane);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ir = 16 * j + 4 * gq + q;
    const uint32_t g = ir < n ? (uint32_t)list[ir] : 0u;
    const uint32_t f = ir < n ? 0u : kFar;
    uint32_t vo = (g * CB3 + vb) | f;
    asm("" : "+v"(vo));  // one load at one address per row
    T.v.va[q] = ld32(rv, vo);
  }
  // this lane's norm row, 4gq + (lane & 3)
  const int in_ = 16 * j + 4 * gq + (lane & 3);
  uint32_t no = in_ < n ? (uint32_t)list[in_] * 4u : kFar;
  T.k.kn = __uint_as_float(ld32(rkn, no));
  T.v.vn = __uint_as_float(ld32(rvn, no));
}

// Top-beta of the scores (0 < beta < ng) by the whole work-group, as a
// bitmap of the selected groups in bits (LDS, zero on entry); hist (zero on
// entry), cand and *nc are LDS scratch.  A 256-bucket histogram over [lo,
// lo + 256 / bscale] (any bounds of the scores) places the beta-th largest
// score in bucket bt; every wave finds bt, and the groups of higher buckets
// are taken.  Wave 0 then ranks the groups of bucket bt exactly by (score
// descending, index ascending) and takes the first `need`; with more than
// kCandCap groups in bt (heavy exact ties) it runs a radix select over all
// scores instead.  The same barriers run on every path; the bitmap is
// complete for wave 0 on return, and for the other waves after their next
// barrier.
template <int NT>
__device__ void select_bits(const uint32_t* tab, int ng, int beta, float lo, float bscale,
                            int* hist, uint2* cand, int* nc, uint32_t* bits, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  for (int g = 4 * tid; g < ng; g += 4 * NT) {
    const f32x4 s = scores4(tab, g);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (g + e < ng) atomicAdd(&hist[score_bucket(fkey(s[e]), lo, bscale)], 1);
  }
  lds_barrier();
  int bt, need;
  hist_threshold(hist, beta, lane, bt, need);
  const int nb = __builtin_amdgcn_readfirstlane(hist[bt]);
  const bool fast = nb <= kCandCap;
  if (fast) {
    for (int g = 4 * tid; g < ng; g += 4 * NT) {
      const f32x4 s = scores4(tab, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (g + e >= ng) break;
        const uint32_t k = fkey(s[e]);
        const int b = score_bucket(k, lo, bscale);
        if (b > bt) atomicOr(&bits[(g + e) >> 5], 1u << ((g + e) & 31));
        if (b == bt) cand[atomicAdd(nc, 1)] = make_uint2((uint32_t)(g + e), k);
      }
    }
  }
  lds_barrier();
  if (wave != 0) return;
  if (fast) {
    for (int i0 = 0; i0 < nb; i0 += 64) {
      const uint2 me = i0 + lane < nb ? cand[i0 + lane] : make_uint2(0u, 0u);
      int rank = 0;
      for (int j = 0; j < nb; ++j) {
        const uint2 o = cand[j];
        rank += (o.y > me.y) || (o.y == me.y && o.x < me.x);
      }
      if (i0 + lane < nb && rank < need) atomicOr(&bits[me.x >> 5], 1u << (me.x & 31));
    }
  } else {
    auto key = [&](int g) {
      return fkey(*reinterpret_cast<const float*>(reinterpret_cast<const char*>(tab) + score_addr(g)));
    };
    int nd;
    const uint32_t kth = radix_kth_f(key, ng, beta, hist, lane, nd);
    int eq_before = 0;
    for (int g0 = 0; g0 < ng; g0 += 64) {
      const int g = g0 + lane;
      const uint32_t k = g < ng ? key(g) : 0u;
      const bool eq = g < ng && k == kth;
      int n_eq;
      const int eq_excl = wave_excl_scan(eq ? 1 : 0, lane, n_eq);
      if ((g < ng && k > kth) || (eq && eq_before + eq_excl < nd))
        atomicOr(&bits[g >> 5], 1u << (g & 31));
      eq_before += n_eq;
    }
  }
  wave_lds_sync();
}

// The one-launch step's small LDS arrays after the static table: [qf]
// [record offsets][selection list][histogram][threshold-bucket groups]
// [selection bitmap].
struct FusedLayout {
  int qf, recoff, sel, hist, cand, bits, end;
};
template <int D, int N, int NW>
__host__ __device__ inline FusedLayout fused_layout(int beta) {
  FusedLayout L;
  L.qf = 0;
  L.recoff = L.qf + kMaxG * kQS<D> * 4;
  L.sel = L.recoff + ((tok_slots<N, NW, FusedCfg<NW>::TD>(beta) * 4 + 15) & ~15);
  L.hist = L.sel + ((max(beta, 1) * 4 + 15) & ~15);
  L.cand = L.hist + 256 * 4;
  L.bits = L.cand + kCandCap * 8;
  L.end = L.bits + (kFusedMaxGroups / 32) * 4;
  return L;
}

// the register budget of FusedCfg<NW> so that two work-groups (the LDS
// limit) fit on a CU
template <int D, int N, bool MEAN, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FusedCfg<NW>::WPE)))
void step_kernel(SumArgs ra, TokArgs ta) {
  constexpr int NT = NW * 64, SD = FusedCfg<NW>::SD, TD = FusedCfg<NW>::TD;
  extern __shared__ __align__(16) char smem[];
  __shared__ __align__(16) uint32_t tab[kTabBytes / 4];
  __shared__ uint32_t s_vsb[kMaxG * (D / 8)];
  __shared__ float s_lo[NW], s_hi[NW];
  __shared__ int s_nc;
  constexpr int CB3 = 3 * D / 8;
  constexpr int LPV = D / 8;
  const FusedLayout FL = fused_layout<D, N, NW>(ra.beta);
  float* qf = reinterpret_cast<float*>(smem + FL.qf);
  int32_t* recoff = reinterpret_cast<int32_t*>(smem + FL.recoff);
  int32_t* sel = reinterpret_cast<int32_t*>(smem + FL.sel);
  int* hist = reinterpret_cast<int*>(smem + FL.hist);
  uint2* cand = reinterpret_cast<uint2*>(smem + FL.cand);
  uint32_t* bits = reinterpret_cast<uint32_t*>(smem + FL.bits);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int c = lane & 15, gq = lane >> 4;
  const int unit = blockIdx.x;
  const int kvh = unit % ra.Hkv;
  const int ng = ra.ng, beta = ra.beta;
  const uint32_t lane4 = (uint32_t)(lane & 31) << 2;
  const uint32_t* tabh = tab + kHiHalf / 4;  // the high halves
  const uint32_t rec = (uint32_t)(N * (D + 8));
  // the summary partial is empty when every group is fetched; the router
  // runs whenever it is not
  const bool stream = beta < ng;
  const int n_tiles = stream ? (ng + 15) >> 4 : 0;

  const rsrc_t rk = make_rsrc(ra.l2k + (size_t)unit * ra.ngs * CB3, (uint32_t)ng * CB3);
  const rsrc_t rkn = make_rsrc(ra.l2k_n + (size_t)unit * ra.ngs, (uint32_t)ng * 4);
  const rsrc_t rv = make_rsrc(ra.l2v + (size_t)unit * ra.ngs * CB3, (uint32_t)ng * CB3);
  const rsrc_t rvn = make_rsrc(ra.l2v_n + (size_t)unit * ra.ngs, (uint32_t)ng * 4);
  const TokBufs TB = tok_bufs<D, N>(ta, unit);
  const int n1t = (ta.n1 + 15) / 16;

  // (0) global loads first: the set-up inputs and this wave's first summary
  // tiles, whose latency the set-up below overlaps
  // the tables are built by the first 512 threads (8 waves)
  TabIn tin{};
  if (tid < 512) tin = load_tab_in(ta.cb4, ra.cb3, tid);
  QueryIn qin;
  load_query<D>(ra.q + (size_t)unit * ra.G * D, ra.k_signs + kvh * (D / 32), ra.G, tid, qin);
  const uint32_t vsb =
      (tid < kMaxG * LPV) ? sign_byte(ta.v_signs + kvh * (D / 32), tid % LPV) : 0u;
  auto load_tile = [&](int t, SumTile& T) {
    load_keys<D>(rk, rkn, t, lane, T.k);
    load_vals<D>(rv, rvn, t, lane, T.v);
  };
  SumTile ft[SD];
#pragma unroll
  for (int j = 0; j < SD - 1; ++j) load_tile(wave + j * NW, ft[j]);

  for (int s = beta + tid; s < tok_slots<N, NW, TD>(beta); s += NT) recoff[s] = (int32_t)kFar;
  for (int b = tid; b < 256; b += NT) hist[b] = 0;
  if (tid < kFusedMaxGroups / 32) bits[tid] = 0u;
  if (tid == 0) s_nc = 0;
  if (tid < kMaxG * LPV) s_vsb[tid] = vsb;
  if (tid < 512) build_tables(tab, tin, tid);
  rotate_query<D>(qin, ra.scale * rsqrtf((float)D), qf, tid);
  lds_barrier();

  // (1) the summary stream
  // wave priorities: the stream 2, the selection 3 (the work-group waits on
  // it), the tokens 1, the epilogue 0; where two work-groups share a CU, the
  // one that is behind gets the issue slots first
  __builtin_amdgcn_s_setprio(2);
  Softmax<D> st;
  st.init(kNegInf);
  float lo = kPosInf, hi = kNegInf;
  if (stream) {
    half8 qb[D / 32];
    router_operands_pad<D>(qf, lane, ra.G, MEAN, qb);
    const float inv_g = 1.f / (float)ra.G;
    const uint32_t vsh = val_shift<D>(lane);
    const int last = n_tiles - 1;
    const int tail = ng - 16 * last - 4 * gq;  // rows of the last tile for this lane
    const int m = skew_rounds<NW, SD>(n_tiles);
    const int n_iters = skew_iters<NW>(n_tiles, m, wave);
    pipeline<SD>(
        n_iters, ft,
        [&](int i, SumTile& T) { load_tile(skew_tile<NW>(i, m, wave, n_tiles), T); },
        [&](int i, const SumTile& T) {
          const int t = skew_tile<NW>(i, m, wave, n_tiles);
          uint32_t kw[3];
          key_bits<D>(T.k.kw, lane, kw);
          const f32x4 lg4 = mul_rows(qk3_exact<D>(kw, qb, tabh, lane4), T.k.kn);
          f32x4 s = row_agg<MEAN>(lg4);
          if constexpr (MEAN) s *= inv_g;
          // rows past the last group score 0 (norm 0): still bounds of the scores
          lo = min3f(min3f(lo, s[0], s[1]), s[2], s[3]);
          hi = max3f(max3f(hi, s[0], s[1]), s[2], s[3]);
          if (c == 0) {  // scores 16t + 4gq .. +3 (see score_addr)
            const uint32_t sa = ((uint32_t)(kScoreBlock + (t >> 1)) << 8) + 64u * (t & 1);
            *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(tab) + kHiHalf + sa + 16 * gq) = s;
          }
          float lg[4] = {lg4[0], lg4[1], lg4[2], lg4[3]};
          if (t == last) {  // wave-uniform: rows past the last group weigh nothing
            // (the empty asm keeps this a branch: selects would cost every tile)
            asm volatile("");
#pragma unroll
            for (int r = 0; r < 4; ++r) lg[r] = r < tail ? lg[r] : kNegInf;
          }
          float p[4], w[4];
          st.update(lg, p);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            st.l += p[r];
            w[r] = p[r] * row_norm(T.v.vn, r);
          }
          pv3_tab<D>(T.v.va, vsh, weight_operand(w, lane), lane4, tabh, st.O);
        });
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
  }
  // The summary bias shifts every summary logit and the reference alike: the
  // stream took the weights without it, so it joins m now, before any token
  // comes in, and the subtracted logits carry it.
  st.m += ra.bias;
  st.mL = st.m * kLog2e;
  st.mth = st.m + kLazy;
  // this wave's first L1 token tiles (they need no selection) load during
  // the selection
  TokTile tt[TD];
#pragma unroll
  for (int j = 0; j < TD - 1; ++j)
    if (wave + j * NW < n1t)  // wave-uniform
      load_tok_at<D, N>(TB, wave + j * NW, n1t, ta.n1, kFar, kFar, lane, tt[j]);
  lds_barrier();  // the scores are complete

  // (2) the selection, as a bitmap, then in ascending order
  __builtin_amdgcn_s_setprio(3);
  if (beta > 0 && beta < ng) {
    lo = kPosInf;
    hi = kNegInf;
    for (int w = 0; w < NW; ++w) {
      lo = fminf(lo, s_lo[w]);
      hi = fmaxf(hi, s_hi[w]);
    }
    const float bs = 256.f / (hi - lo);
    const float bscale = (hi > lo && __builtin_isfinite(bs)) ? bs : 0.f;
    select_bits<NT>(tab, ng, beta, lo, bscale, hist, cand, &s_nc, bits, tid);
    if (wave == 0) {
      int32_t* idx = ra.idx ? ra.idx + (size_t)unit * beta : nullptr;
      int pos0 = 0;
      for (int w0 = 0; w0 < (ng + 31) >> 5; w0 += 64) {
        const int wd = w0 + lane;
        uint32_t b = wd < (ng + 31) >> 5 ? bits[wd] : 0u;
        int total;
        int pos = pos0 + wave_excl_scan(__popc(b), lane, total);
        while (b) {
          const int g = 32 * wd + __ffs(b) - 1;
          if (pos < beta) {  // exactly beta bits are set; the test keeps the lists in bounds
            sel[pos] = g;
            recoff[pos] = (int32_t)((uint32_t)g * rec);
            if (idx) idx[pos] = g;
          }
          ++pos;
          b &= b - 1u;
        }
        pos0 += total;
      }
    }
  } else if (beta > 0) {  // every group fetched
    int32_t* idx = ra.idx ? ra.idx + (size_t)unit * beta : nullptr;
    for (int g = tid; g < beta; g += NT) {
      recoff[g] = (int32_t)((uint32_t)g * rec);
      if (idx) idx[g] = g;
    }
  }
  lds_barrier();  // the record offsets and the selection list are visible

  // (3) The fetched groups' summaries come out first: 16 a tile, subtracted
  // with the stream's own logits (the same code and operands).  Then one
  // pipeline over the L1 tiles and the fetched tokens.
  __builtin_amdgcn_s_setprio(1);
  const int ntc = (stream && beta > 0) ? (beta + 15) / 16 : 0;
  const int nft = (N == 16) ? beta : (beta + 1) / 2;
  const int total = n1t + nft;
  const int iters = wave_iters<NW>(total, wave);
  auto tile_of = [&](int i) { return i < iters ? wave + i * NW : total + wave + NW * (i - iters); };
  SumTile ct;
  if (wave < ntc) load_sum_list<D>(rk, rkn, rv, rvn, sel, beta, wave, lane, ct);
#pragma unroll
  for (int j = 0; j < TD - 1; ++j)
    if (!(wave + j * NW < n1t))  // wave-uniform: the fetched tiles among the first
      load_tok<D, N>(TB, recoff, tile_of(j), n1t, ta.n1, lane, tt[j]);
  if (wave < ntc) {
    half8 qb[D / 32];
    router_operands_pad<D>(qf, lane, ra.G, MEAN, qb);
    const uint32_t vsh = val_shift<D>(lane);
    for (int j = wave; j < ntc; j += NW) {
      if (j != wave) load_sum_list<D>(rk, rkn, rv, rvn, sel, beta, j, lane, ct);
      uint32_t kw[3];
      key_bits<D>(ct.k.kw, lane, kw);
      const f32x4 lg4 = mul_rows(qk3_exact<D>(kw, qb, tabh, lane4), ct.k.kn);
      float lg[4], p[4], w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lg[r] = (16 * j + 4 * gq + r < beta) ? lg4[r] + ra.bias : kNegInf;
      st.update(lg, p);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st.l -= p[r];
        w[r] = -p[r] * row_norm(ct.v.vn, r);
      }
      pv3_tab<D>(ct.v.va, vsh, weight_operand(w, lane), lane4, tabh, st.O);
    }
  }
  {
    half8 qh[D / 32], ql[D / 32];
    query_operands<D>(qf, lane, qh, ql);
    const int ragged = (ta.n1 & 15) ? n1t - 1 : -1;
    const int half = (N == 8 && (beta & 1)) ? total - 1 : -1;
    pipeline<TD>(
        iters, tt,
        [&](int i, TokTile& T) { load_tok<D, N>(TB, recoff, tile_of(i), n1t, ta.n1, lane, T); },
        [&](int i, const TokTile& T) {
          const int t = tile_of(i);
          consume_tok<D>(
              T, t == ragged || t == half,
              [&](float (&lg)[4]) { mask_rows<N>(lg, t, n1t, ta.n1, beta, recoff, lane); }, qh,
              tab, lane, lane4, st);
        });
  }
  lds_barrier();  // the tables are no longer needed: reuse as scratch

  // (4) combine, normalise, inverse V rotation, output
  __builtin_amdgcn_s_setprio(0);
  float* scratch = reinterpret_cast<float*>(tab);
  // head stride of the scratch: kMaxG, or G with 16 waves (so that 17
  // partials and the output fit in the 64 KB region; the launch checks it)
  const int gs = NW > 8 ? ra.G : kMaxG;
  float* mine = scratch + NW * gs * (D + 2);
  combine_waves<D, NW>(st, ra.G, scratch, mine, tid, gs);
  float* o = mine + gs * (D + 2);
  for (int k = tid; k < ra.G * D; k += NT) {
    const int h = k / D, e = k % D;
    const float l = mine[h * (D + 2) + 1];
    o[k] = l > 0.f ? mine[h * (D + 2) + 2 + e] / l : 0.f;
  }
  lds_barrier();
  if (tid < kMaxG * LPV) {
    const int h = tid / LPV, sub = tid % LPV;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (h < ra.G) ? o[h * D + 8 * sub + k] : 0.f;
    fwht8xlanes<LPV>(v, sub);
    if (h < ra.G) {
      const uint32_t sb = s_vsb[tid];
      const float sc = rsqrtf((float)D);
      float* dst = ta.out + ((size_t)unit * ra.G + h) * D + 8 * sub;
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = flip(v[k] * sc, (sb >> k) & 1u);
    }
  }
}

// ------------------------------------------------------ split decode step ---
//
// For few units, or more summaries than the one-launch step holds on chip,
// the step runs as four launches that spread every unit over many
// work-groups (no cross-work-group synchronisation inside a launch; the
// workspace carries the hand-overs):
//   split_scores_kernel  chunk c of a unit's summary keys: per-head logits
//                        (the router arithmetic above) and each group's
//                        router key, both to the workspace
//   split_select_kernel  one work-group per unit: histogram of the keys,
//                        the exact top-beta (select_wave), the selection and
//                        its bitmap
//   split_attend_kernel  two kinds of work-groups: summary-value chunks (the
//                        unfetched summaries, logits from the workspace) and
//                        token chunks (L1 and fetched tiles); each writes one
//                        partial (m, l, O) per head
//   split_merge_kernel   one work-group per unit: log-sum-exp merge of the
//                        partials, inverse V rotation, output

constexpr int kScoreWaves = 2;                 // scores kernel: 2 waves, one tile each
constexpr int kScoreTiles = kScoreWaves;

struct SplitPlan {
  int ngp, words, n_vt, n_tt;   // groups padded to 16; bitmap words; value / token tiles
  int s1, sv, st, vt, tt;       // score chunks; value / token chunks; tiles per chunk
};
__host__ __device__ inline SplitPlan split_plan(int units, int n1, int ng, int beta, int N) {
  SplitPlan p;
  p.ngp = (ng + 15) & ~15;
  p.words = (p.ngp + 31) / 32;
  p.n_vt = p.ngp / 16;
  p.n_tt = (n1 + 15) / 16 + (N == 16 ? beta : (beta + 1) / 2);
  p.s1 = (p.n_vt + kScoreTiles - 1) / kScoreTiles;
  // about 16 attend work-groups per unit, 2 .. 16 tiles each; the chunks
  // depend on the unit's own sizes only, so a unit's result does not depend
  // on the batch it is run in
  (void)units;
  int per = (p.n_vt + p.n_tt + 15) / 16;
  per = per < 2 ? 2 : (per > 16 ? 16 : per);
  p.vt = p.tt = per;
  p.sv = (p.n_vt + per - 1) / per;
  p.st = (p.n_tt + per - 1) / per;
  if (p.st < 1) p.st = 1;
  return p;
}

struct SplitArgs {
  SumArgs r;        // router inputs (q, L2, signs, cb3, scale, bias, agg, G, Hkv, ng, beta, ngs)
  TokArgs t;        // attend inputs
  SplitPlan p;
  float* lgt;       // [units][G][ngp] per-head logits
  uint32_t* keys;   // [units][ngp] router keys
  float* rn;        // [units][s1] largest key norm per score chunk
  uint32_t* bits;   // [units][words] selection bitmap
  int32_t* sel;     // [units][beta] selection
  int32_t* idx_out; // optional [units][beta]
  float* parts;     // [units][sv + st][G][D+2]
  int chunk0, nchunk;  // split_attend_kernel: chunks chunk0 .. chunk0 + nchunk - 1 of each unit
};

// Scores of 16 * kScoreTiles summaries of one unit: logits to a.lgt, router
// keys to a.keys (EXACT: the three-term router, scores also to scores_out).
template <int D, bool EXACT>
__global__ __launch_bounds__(64 * kScoreWaves) void split_scores_kernel(SplitArgs a) {
  constexpr int CB3 = 3 * D / 8;
  __shared__ __align__(16) uint32_t s_lut3[64 * kNC3];
  __shared__ __align__(16) uint32_t s_lut3lo[EXACT ? 64 * kNC3 : 4];
  __shared__ __align__(16) float s_qf[kMaxG * kQS<D>];
  __shared__ float s_cb[8];
  __shared__ float s_rnw[kScoreWaves];
  const SumArgs& r = a.r;
  const int unit = blockIdx.x / a.p.s1, chunk = blockIdx.x % a.p.s1;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int kvh = unit % r.Hkv;
  const uint32_t lane4 = (uint32_t)(lane & 31) << 2;
  const int c = lane & 15, gq = lane >> 4;
  const rsrc_t rk = make_rsrc(r.l2k + (size_t)unit * r.ngs * CB3, (uint32_t)r.ng * CB3);
  const rsrc_t rkn = make_rsrc(r.l2k_n + (size_t)unit * r.ngs, (uint32_t)r.ng * 4);
  const int t = chunk * kScoreTiles + wave;  // this wave's tile
  KeyTile kt;
  load_keys<D>(rk, rkn, t, lane, kt);
  QueryIn qin;
  // the query rows are rotated by the first 8 * D / 8 threads: with two
  // waves and D = 128 that is all of them; each thread does its share
  const float cbv = (tid < 8) ? r.cb3[tid] : 0.f;
  if (tid < 8) s_cb[tid] = cbv;
  for (int base = 0; base < kMaxG * (D / 8); base += 64 * kScoreWaves) {
    load_query<D>(r.q + (size_t)unit * r.G * D, r.k_signs + kvh * (D / 32), r.G, base + tid, qin);
    rotate_query<D>(qin, r.scale * rsqrtf((float)D), s_qf, base + tid);
  }
  lds_barrier();
  for (int e = tid; e < 64 * 8; e += 64 * kScoreWaves) {
    build_lut3(s_lut3, s_cb, e);
    if constexpr (EXACT) build_lut3_lo(s_lut3lo, s_cb, e);
  }
  half8 qb[D / 32];
  router_operands<D>(s_qf, lane, qb);
  lds_barrier();
  uint32_t kw[3];
  key_bits<D>(kt.kw, lane, kw);
  f32x4 lg = mul_rows(qk3<D, EXACT>(kw, qb, s_lut3, s_lut3lo, lane4), kt.kn);
  const float rn = wave_max(fmaxf(kt.kn, 0.f));
  const int g0 = 16 * t + 4 * gq;
  const bool live = t < a.p.n_vt;  // wave-uniform: the last chunk may have a tile past the end
  if (live && c < r.G) {
    float* dst = a.lgt + ((size_t)unit * r.G + c) * a.p.ngp + g0;
    *reinterpret_cast<f32x4*>(dst) = lg;
  }
  // router score of rows g0 .. g0+3: max (or mean) over the lanes c < G of
  // this row of 16 lanes
  const bool mean = r.agg != HSQ_AGG_MAX;
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = (c < r.G) ? lg[i] : (mean ? 0.f : kNegInf);
    if (mean) {
      x = group_sum<16>(x) * (1.f / (float)r.G);
    } else {
      x = fmaxf(x, dpp_f<0xb1>(x));
      x = fmaxf(x, dpp_f<0x4e>(x));
      x = fmaxf(x, dpp_f<0x141>(x));
      x = fmaxf(x, dpp_f<0x140>(x));
    }
    sc[i] = x;
  }
  if (live && c == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = g0 + i < r.ng;
      a.keys[(size_t)unit * a.p.ngp + g0 + i] = ok ? fkey(sc[i]) : 0u;
      if (EXACT && r.scores_out && ok) r.scores_out[(size_t)unit * r.ng + g0 + i] = sc[i];
    }
  }
  if (lane == 0) s_rnw[wave] = rn;
  lds_barrier();
  if (tid == 0) {
    float m = 0.f;
    for (int w = 0; w < kScoreWaves; ++w) m = fmaxf(m, s_rnw[w]);
    a.rn[(size_t)unit * a.p.s1 + chunk] = m;
  }
}

// Selection of one unit from its router keys (eight waves: keys to LDS and
// the histogram; then one wave selects).  LDS: [keys ngp][hist 256][cand 64]
// [fmask words][qf].
template <int D, bool EXACT>
__global__ __launch_bounds__(kThreads) void split_select_kernel(SplitArgs a) {
  constexpr int CB3 = 3 * D / 8;
  extern __shared__ __align__(16) char smem[];
  __shared__ float s_cb[8];
  __shared__ float s_qn[kMaxG];
  __shared__ float s_lo[kWaves], s_hi[kWaves];
  const SumArgs& r = a.r;
  const int unit = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int kvh = unit % r.Hkv;
  const SplitPlan& p = a.p;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
  int* hist = reinterpret_cast<int*>(keys + ((p.ngp + 31) & ~31));
  uint2* cand = reinterpret_cast<uint2*>(hist + 256);
  uint32_t* fmask = reinterpret_cast<uint32_t*>(cand + 64);
  float* qf = reinterpret_cast<float*>(fmask + ((p.words + 3) & ~3));
  const rsrc_t rk = make_rsrc(r.l2k + (size_t)unit * r.ngs * CB3, (uint32_t)r.ng * CB3);
  const rsrc_t rkn = make_rsrc(r.l2k_n + (size_t)unit * r.ngs, (uint32_t)r.ng * 4);
  const float cbv = (tid < 8) ? r.cb3[tid] : 0.f;
  QueryIn qin;
  load_query<D>(r.q + (size_t)unit * r.G * D, r.k_signs + kvh * (D / 32), r.G, tid, qin);
  float lo = kPosInf, hi = kNegInf;
  const uint32_t* kin = a.keys + (size_t)unit * p.ngp;
  for (int g = tid; g < p.ngp; g += kThreads) {
    const uint32_t k = kin[g];
    keys[g] = k;
    if (g < r.ng) {
      const float f = key_float(k);
      lo = fminf(lo, f);
      hi = fmaxf(hi, f);
    }
  }
  for (int b = tid; b < 256; b += kThreads) hist[b] = 0;
  for (int w = tid; w < p.words; w += kThreads) {
    const int left = r.ng - 32 * w;
    fmask[w] = (r.beta >= r.ng) ? (left >= 32 ? 0xffffffffu : (left <= 0 ? 0u : ((1u << left) - 1u)))
                                : 0u;
    a.bits[(size_t)unit * p.words + w] = 0u;
  }
  if (tid < 8) s_cb[tid] = cbv;
  rotate_query<D>(qin, r.scale * rsqrtf((float)D), qf, tid, s_qn);
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
  }
  __syncthreads();  // also orders the bitmap's zeroing before its atomics below
  lo = kPosInf;
  hi = kNegInf;
  for (int w = 0; w < kWaves; ++w) {
    lo = fminf(lo, s_lo[w]);
    hi = fmaxf(hi, s_hi[w]);
  }
  const float bscale = (hi > lo) ? 256.f / (hi - lo) : 0.f;
  const bool hsel = r.beta > 0 && r.beta < r.ng;
  if (hsel)
    for (int g = tid; g < r.ng; g += kThreads) atomicAdd(&hist[score_bucket(keys[g], lo, bscale)], 1);
  lds_barrier();
  if (wave != 0) return;
  float bnd = 0.f;
  if constexpr (!EXACT) {
    if (hsel) {
      float rmax = 0.f, qn = 0.f;
      for (int k = lane; k < p.s1; k += 64) rmax = fmaxf(rmax, a.rn[(size_t)unit * p.s1 + k]);
      rmax = wave_max(rmax);
      for (int h = 0; h < r.G; ++h) qn = fmaxf(qn, s_qn[h]);
      const float cl = lane < 8 ? s_cb[lane] : 0.f;
      const float dl = wave_max(fabsf(cl - (float)(_Float16)cl));
      const float cm = wave_max(fabsf(cl));
      bnd = rmax * qn * (dl + cm * 0x1p-14f) * 1.0625f;
    }
  }
  SelIo io;
  io.keys = keys; io.hist = hist; io.cand = cand; io.fmask = fmask;
  io.words = p.words; io.ng = r.ng; io.beta = r.beta; io.G = r.G;
  io.lo = lo; io.bscale = bscale; io.bnd = bnd; io.hsel = hsel;
  io.mean = r.agg != HSQ_AGG_MAX;
  io.rk = rk; io.rkn = rkn; io.qf = qf; io.cb = s_cb;
  io.idx = a.sel + (size_t)unit * r.beta;
  io.recoff = nullptr; io.rec = 0u;
  io.bits = a.bits + (size_t)unit * p.words;
  const int nsel = select_wave<D, EXACT>(io, lane);
  if (a.idx_out)
    for (int i = lane; i < nsel; i += 64) a.idx_out[(size_t)unit * r.beta + i] = (int32_t)keys[i];
}

// Attend work-groups.  blockIdx: unit * (sv + st) + k; k < sv: summary-value
// chunk k (tiles k * vt ..), else token chunk k - sv (tiles k - sv, with
// stride st, of the unit's L1 and fetched tiles).  Each writes its partial
// (m, l, O) per head to parts[unit][k].
template <int D, int N, typename TT = TokTile>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void split_attend_kernel(SplitArgs a) {
  extern __shared__ __align__(16) char smem[];
  __shared__ __align__(16) uint32_t s_tab[kLut4Bytes / 4];
  __shared__ float s_cb[16];
  const SplitPlan& p = a.p;
  const int per = p.sv + p.st;
  const int unit = blockIdx.x / a.nchunk, k = a.chunk0 + blockIdx.x % a.nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int G = a.r.G;
  float* part = a.parts + ((size_t)unit * per + k) * G * (D + 2);
  if (k < p.sv) {
    // summary values of tiles k * vt .. (k + 1) * vt - 1, unfetched rows only
    constexpr int CB3 = 3 * D / 8;
    const SumArgs& r = a.r;
    const rsrc_t rv = make_rsrc(r.l2v + (size_t)unit * r.ngs * CB3, (uint32_t)r.ng * CB3);
    const rsrc_t rvn = make_rsrc(r.l2v_n + (size_t)unit * r.ngs, (uint32_t)r.ng * 4);
    const int t0 = k * p.vt, nt = min(p.vt, p.n_vt - t0);
    const int iters = wave_iters(nt, wave);
    constexpr int K = kValDepth;
    auto tile = [&](int i) { return i < iters ? t0 + wave + i * kWaves : p.n_vt + wave; };
    ValTile vt[K];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) load_vals<D>(rv, rvn, tile(j), lane, vt[j]);
    const float cbv = (tid < 8) ? r.cb3[tid] : 0.f;
    if (tid < 8) s_cb[tid] = cbv;
    lds_barrier();
    build_lut3(s_tab, s_cb, tid);
    lds_barrier();
    const int c = lane & 15, gq = lane >> 4, hcol = min(col_head(c), G - 1);
    const uint32_t lane4 = (uint32_t)(lane & 31) << 2;
    const float* lrow = a.lgt + ((size_t)unit * G + hcol) * p.ngp + 4 * gq;
    const uint32_t* bw = a.bits + (size_t)unit * p.words;
    const uint32_t vsh = val_shift<D>(lane);
    Softmax<D> st;
    st.init(kNegInf);
    pipeline<K>(
        iters, vt, [&](int i, ValTile& V) { load_vals<D>(rv, rvn, tile(i), lane, V); },
        [&](int i, const ValTile& V) {
          const int t = tile(i);
          const f32x4 lg4 = *reinterpret_cast<const f32x4*>(lrow + 16 * t);
          const uint32_t fw = bw[(16 * t + 4 * gq) >> 5] >> ((16 * t + 4 * gq) & 31);
          float lg[4], pw[4];
          bool live[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            live[rr] = 16 * t + 4 * gq + rr < r.ng && !((fw >> rr) & 1u);
            lg[rr] = live[rr] ? lg4[rr] : kNegInf;
          }
          st.update(lg, pw);
          float w[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            // a masked row weighs 0 (also while no live row has set the
            // reference, where exp(-inf - -inf) is not a number)
            pw[rr] = live[rr] ? pw[rr] : 0.f;
            st.l += pw[rr];
            w[rr] = pw[rr] * row_norm(V.vn, rr);
          }
          pv3<D>(V.va, vsh, weight_operand(w, lane), lane4, s_tab, st.O);
        });
    st.m += r.bias;
    lds_barrier();
    combine_waves<D>(st, G, reinterpret_cast<float*>(s_tab), part, tid);
    return;
  }
  // token chunk: the attend body over tiles (k - sv), (k - sv) + st, ...
  const TokArgs& ta = a.t;
  const int kvh = unit % ta.Hkv;
  AttendLds L;
  L.lut4 = s_tab;
  L.qf = reinterpret_cast<float*>(smem);
  L.part = nullptr;
  L.recoff = reinterpret_cast<int32_t*>(L.qf + kMaxG * kQS<D>);
  L.cb = s_cb;
  L.vsb = nullptr;
  const size_t rec = (size_t)N * (D + 8);
  const float cbv = (tid < 16) ? ta.cb4[tid] : 0.f;
  QueryIn qin;
  load_query<D>(ta.q + (size_t)unit * G * D, ta.k_signs + kvh * (D / 32), G, tid, qin);
  // record of slot s: group sel[s] of the archive, or slot s of the staging
  // buffer when the records were gathered there (l3_staged)
  const int32_t* sel = a.sel + (size_t)unit * ta.beta;
  for (int s = tid; s < tok_slots<N>(ta.beta); s += kThreads) {
    const int g = s < ta.beta ? sel[s] : -1;
    const bool ok = g >= 0 && g < ta.ng;
    const uint32_t r = ta.l3_staged ? (uint32_t)s : (uint32_t)g;
    L.recoff[s] = ok ? (int32_t)(r * (uint32_t)rec) : (int32_t)kFar;
  }
  if (tid < 16) s_cb[tid] = cbv;
  // the variant tiles (pre-RoPE rows, TQ-QKV sketches) as in token_kernel
  L.uf = reinterpret_cast<float*>(L.recoff + ((tok_slots<N>(ta.beta) + 3) & ~3));
  L.qm = reinterpret_cast<_Float16*>(L.uf);
  if constexpr (std::is_same_v<TT, TokTileK>) stage_query_model<D>(qin, ta.scale, L.qm, tid);
  rotate_query<D>(qin, ta.scale * rsqrtf((float)D), L.qf, tid);
  lds_barrier();
  constexpr int TD = std::is_same_v<TT, TokTile> ? kTokDepth : kTokDepth - 1;
  TT tt[TD];
  attend_unit<D, N, TT, TD>(ta, L, tt, false, nullptr, nullptr, unit, k - p.sv, p.st, part);
}

// Merge of one unit's partials and the inverse V rotation (8 * D / 8
// threads: head h, 8 coordinates per thread).
template <int D>
__global__ __launch_bounds__(kMaxG * (D / 8)) void split_merge_kernel(SplitArgs a) {
  constexpr int LPV = D / 8;
  const int unit = blockIdx.x, tid = threadIdx.x, h = tid / LPV, sub = tid % LPV;
  const int G = a.r.G, per = a.p.sv + a.p.st;
  const int kvh = unit % a.t.Hkv;
  if (h >= G) return;  // whole row groups: the lanes of one head stay together
  const float* base = a.parts + (size_t)unit * per * G * (D + 2) + h * (D + 2);
  float M = kNegInf;
  for (int k = 0; k < per; ++k) M = fmaxf(M, base[(size_t)k * G * (D + 2)]);
  float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < per; ++k) {
    const float* pk = base + (size_t)k * G * (D + 2);
    const float m = pk[0];
    const float w = (m == kNegInf) ? 0.f : __expf(m - M);
    L += w * pk[1];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += w * pk[2 + 8 * sub + e];
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= inv;
  fwht8xlanes<LPV>(o, sub);
  const uint32_t sb = sign_byte(a.t.v_signs + kvh * (D / 32), sub);
  const float sc = rsqrtf((float)D);
  float* dst = a.t.out + ((size_t)unit * G + h) * D + 8 * sub;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = flip(o[e] * sc, (sb >> e) & 1u);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t summary_smem(int D, const StepShape& s) {
  const size_t body =
      (size_t)route_layout(s.G, s.n_groups, s.beta, kMaxG * (D + 4) * 4 + 64 * 16).end;
  const size_t comb = (size_t)kWaves * kMaxG * (D + 2) * 4;
  return std::max(body, comb);
}

// variant: the region after the record offsets (TQ-QKV u rows, or the
// pre-RoPE unrotated query)
size_t token_smem(int D, const StepShape& s, bool variant = false) {
  const int slots = s.group_n == 16 ? tok_slots<16>(s.beta) : tok_slots<8>(s.beta);
  return (size_t)kMaxG * (D + 4) * 4 + (size_t)kMaxG * (D + 2) * 4 +
         (size_t)((slots + 3) & ~3) * 4 + (variant ? (size_t)kMaxG * (D + 4) * 4 : 0);
}

// Waves per work-group of the one-launch step: 16 (one work-group per CU)
// for layers of at most kFewUnits units with at least kFewGroups groups (a
// stream long enough to split further) whose epilogue scratch (17 wave
// partials at head stride G, this unit's partial and the output) fits the
// 64 KB table region, else 8 (two work-groups per CU).  Measured: 64 units
// of 2002 groups 34.4 -> 31.2 us with 16 waves; 8 units of 497 groups 18.1
// -> 19.0 us (a short stream gains nothing from more waves).
int fused_waves(const StepShape& s) {
  const size_t scratch = (size_t)(17 * s.G * (s.d + 2) + s.G * (s.d + 2) + s.G * s.d) * 4;
  return (s.B * s.Hkv <= kFewUnits && s.n_groups >= kFewGroups && scratch <= (size_t)kTabBytes)
             ? kFusedWavesFew
             : kFusedWaves;
}

template <int NW>
size_t step_smem_nw(const StepShape& s) {
  if (s.d == 128)
    return (size_t)(s.group_n == 16 ? fused_layout<128, 16, NW>(s.beta).end
                                    : fused_layout<128, 8, NW>(s.beta).end);
  return (size_t)(s.group_n == 16 ? fused_layout<64, 16, NW>(s.beta).end
                                  : fused_layout<64, 8, NW>(s.beta).end);
}

size_t step_smem(const StepShape& s) {
  return fused_waves(s) == kFusedWavesFew ? step_smem_nw<kFusedWavesFew>(s)
                                          : step_smem_nw<kFusedWaves>(s);
}

}  // namespace

int route_lds_ok(const StepShape& s) { return s.G * ((s.n_groups + 15) & ~15) <= kMaxLogits; }

int split_shape(const StepShape& s) {
  return s.n_groups > 0 && (s.B * s.Hkv < kSplitUnits || !route_lds_ok(s));
}

int use_split(const StepShape& s) { return split_shape(s) && !step_fused_ok(s); }

Workspace plan_workspace(const StepShape& s) {
  Workspace w{};
  const int units = s.B * s.Hkv;
  size_t off = 0;
  w.idx_off = off;  off = align256(off + (size_t)units * std::max(s.beta, 1) * 4);
  w.part_off = off; off = align256(off + (size_t)units * s.G * (s.d + 2) * 4);
  if (split_shape(s)) {
    const SplitPlan p = split_plan(units, s.n_l1, s.n_groups, s.beta, s.group_n);
    w.lgt_off = off;   off = align256(off + (size_t)units * s.G * p.ngp * 4);
    w.keys_off = off;  off = align256(off + (size_t)units * p.ngp * 4);
    w.rn_off = off;    off = align256(off + (size_t)units * p.s1 * 4);
    w.bits_off = off;  off = align256(off + (size_t)units * p.words * 4);
    w.parts_off = off; off = align256(off + (size_t)units * (p.sv + p.st) * s.G * (s.d + 2) * 4);
  }
  w.total = off;
  return w;
}

int step_limits_ok(const StepShape& s) {
  const size_t rec = (size_t)s.group_n * (s.d + 8);
  return s.n_groups <= kMaxGroups && (size_t)s.n_groups * rec < 0x7fffffffu &&
         (size_t)s.n_l1 * s.d < 0x7fffffffu;
}

SumArgs sum_args(const StepShape& s, const StepTensors& t) {
  SumArgs a{};
  a.q = t.q; a.l2k = t.l2k; a.l2k_n = t.l2k_n; a.l2v = t.l2v; a.l2v_n = t.l2v_n;
  a.k_signs = t.k_signs; a.cb3 = t.cb3; a.scale = t.scale; a.bias = t.summary_bias;
  a.agg = t.agg; a.Hkv = s.Hkv; a.G = s.G; a.ng = s.n_groups; a.beta = s.beta;
  a.ngs = s.ng_stride > 0 ? s.ng_stride : s.n_groups;
  return a;
}

TokArgs tok_args(const StepShape& s, const StepTensors& t) {
  TokArgs a{};
  a.q = t.q; a.l1k = t.l1k; a.l1k_n = t.l1k_n; a.l1v = t.l1v; a.l1v_n = t.l1v_n;
  a.l3 = t.l3; a.l3_staged = t.l3_staged;
  a.k_signs = t.k_signs; a.v_signs = t.v_signs; a.cb4 = t.cb4; a.scale = t.scale;
  a.Hkv = s.Hkv; a.G = s.G; a.n1 = s.n_l1; a.ng = s.n_groups; a.group_n = s.group_n;
  a.beta = s.beta;
  a.n1s = s.l1_stride > 0 ? s.l1_stride : s.n_l1;
  a.ngs = s.ng_stride > 0 ? s.ng_stride : s.n_groups;
  a.out = t.out;
  return a;
}

template <int D>
hipError_t summary_d(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                     int mode, const int32_t* given, float* scores_out, int32_t* idx_out,
                     hipStream_t st) {
  SumArgs a = sum_args(s, t);
  a.want_topk = (mode & ROUTE_TOPK) ? 1 : 0;
  a.want_partial = (mode & ROUTE_PARTIALS) ? 1 : 0;
  a.given = a.want_topk ? nullptr : given;
  a.scores_out = scores_out;
  a.idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + w.idx_off);
  a.part = reinterpret_cast<float*>(ws + w.part_off);
  if (scores_out)
    hipLaunchKernelGGL((summary_kernel<D, true>), dim3((unsigned)(s.B * s.Hkv)), dim3(kThreads),
                       summary_smem(D, s), st, a);
  else
    hipLaunchKernelGGL((summary_kernel<D, false>), dim3((unsigned)(s.B * s.Hkv)), dim3(kThreads),
                       summary_smem(D, s), st, a);
  return hipGetLastError();
}

SplitArgs split_args(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws) {
  SplitArgs a{};
  a.r = sum_args(s, t);
  a.t = tok_args(s, t);
  a.p = split_plan(s.B * s.Hkv, s.n_l1, s.n_groups, s.beta, s.group_n);
  a.lgt = reinterpret_cast<float*>(ws + w.lgt_off);
  a.keys = reinterpret_cast<uint32_t*>(ws + w.keys_off);
  a.rn = reinterpret_cast<float*>(ws + w.rn_off);
  a.bits = reinterpret_cast<uint32_t*>(ws + w.bits_off);
  a.sel = reinterpret_cast<int32_t*>(ws + w.idx_off);
  a.parts = reinterpret_cast<float*>(ws + w.parts_off);
  return a;
}

size_t select_smem(const SplitPlan& p, int D) {
  return (size_t)((p.ngp + 31) & ~31) * 4 + 256 * 4 + 64 * 8 + (size_t)((p.words + 3) & ~3) * 4 +
         (size_t)kMaxG * (D + 4) * 4;
}

// Scores and selection of the split step (route only when attend is false).
template <int D>
hipError_t split_route_d(const SplitArgs& a, int units, bool exact, hipStream_t st) {
  const SplitPlan& p = a.p;
  if (exact)
    hipLaunchKernelGGL((split_scores_kernel<D, true>), dim3((unsigned)(units * p.s1)),
                       dim3(64 * kScoreWaves), 0, st, a);
  else
    hipLaunchKernelGGL((split_scores_kernel<D, false>), dim3((unsigned)(units * p.s1)),
                       dim3(64 * kScoreWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (exact)
    hipLaunchKernelGGL((split_select_kernel<D, true>), dim3((unsigned)units), dim3(kThreads),
                       select_smem(p, D), st, a);
  else
    hipLaunchKernelGGL((split_select_kernel<D, false>), dim3((unsigned)units), dim3(kThreads),
                       select_smem(p, D), st, a);
  return hipGetLastError();
}

// Attend chunks [k0, k0 + n) of every unit; with merge, then the merge.
template <int D, int N, typename TT = TokTile>
hipError_t split_attend_dn(SplitArgs a, int units, int k0, int n, bool merge, hipStream_t st) {
  a.chunk0 = k0;
  a.nchunk = n;
  if (n > 0) {
    const size_t smem = (size_t)kMaxG * kQS<D> * 4 + (size_t)((tok_slots<N>(a.t.beta) + 3) & ~3) * 4 +
                        (std::is_same_v<TT, TokTile> ? 0 : (size_t)kMaxG * kQS<D> * 4);
    hipLaunchKernelGGL((split_attend_kernel<D, N, TT>), dim3((unsigned)(units * n)),
                       dim3(kThreads), smem, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (merge)
    hipLaunchKernelGGL((split_merge_kernel<D>), dim3((unsigned)units), dim3(kMaxG * (D / 8)), 0,
                       st, a);
  return hipGetLastError();
}

template <int D, int N>
hipError_t split_step_dn(const SplitArgs& a, int units, hipStream_t st) {
  hipError_t e = split_route_d<D>(a, units, false, st);
  if (e != hipSuccess) return e;
  return split_attend_dn<D, N>(a, units, 0, a.p.sv + a.p.st, true, st);
}

// The split step as two calls with work between them (the host-archive
// path gathers the fetched records in between): scores, selection and the
// summary-value chunks; then the token chunks and the merge.
template <int D, int N>
hipError_t split_halves_dn(const SplitArgs& a, int units, bool first, hipStream_t st) {
  if (first) {
    const hipError_t e = split_route_d<D>(a, units, false, st);
    if (e != hipSuccess) return e;
    return split_attend_dn<D, N>(a, units, 0, a.p.sv, false, st);
  }
  if (a.t.kdense) return split_attend_dn<D, N, TokTileK>(a, units, a.p.sv, a.p.st, true, st);
  if (a.t.S) return split_attend_dn<D, N, TokTileQ>(a, units, a.p.sv, a.p.st, true, st);
  return split_attend_dn<D, N>(a, units, a.p.sv, a.p.st, true, st);
}

hipError_t launch_split_step(const StepShape& s, const StepTensors& t, const Workspace& w,
                             char* ws, int32_t* idx_out, hipStream_t st) {
  if (!step_limits_ok(s) || !split_shape(s)) return hipErrorInvalidValue;
  SplitArgs a = split_args(s, t, w, ws);
  a.idx_out = s.beta > 0 ? idx_out : nullptr;
  const int units = s.B * s.Hkv;
  if (s.d == 128)
    return s.group_n == 16 ? split_step_dn<128, 16>(a, units, st)
                           : split_step_dn<128, 8>(a, units, st);
  return s.group_n == 16 ? split_step_dn<64, 16>(a, units, st) : split_step_dn<64, 8>(a, units, st);
}

hipError_t launch_split_half(const StepShape& s, const StepTensors& t, const Workspace& w,
                             char* ws, bool first, int32_t* idx_out, hipStream_t st,
                             const uint16_t* kdense, const QjlKeys* qk) {
  if (!step_limits_ok(s) || !split_shape(s)) return hipErrorInvalidValue;
  if (kdense && qk) return hipErrorInvalidValue;
  SplitArgs a = split_args(s, t, w, ws);
  a.idx_out = s.beta > 0 ? idx_out : nullptr;
  if (!first) {
    a.t.kdense = s.beta > 0 ? kdense : nullptr;
    if (qk) {
      if (!qk->S || (s.n_l1 > 0 && (!qk->l1_sk || !qk->l1_gam)) ||
          (s.beta > 0 && (!qk->l3_sk || !qk->l3_gam)) || t.l3_staged)
        return hipErrorInvalidValue;
      a.t.l1_sk = qk->l1_sk; a.t.l1_gam = qk->l1_gam; a.t.l3_sk = qk->l3_sk;
      a.t.l3_gam = qk->l3_gam; a.t.S = qk->S;
    }
  }
  const int units = s.B * s.Hkv;
  if (s.d == 128)
    return s.group_n == 16 ? split_halves_dn<128, 16>(a, units, first, st)
                           : split_halves_dn<128, 8>(a, units, first, st);
  return s.group_n == 16 ? split_halves_dn<64, 16>(a, units, first, st)
                         : split_halves_dn<64, 8>(a, units, first, st);
}

hipError_t launch_route(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                        int mode, const int32_t* given, float* scores_out, int32_t* idx_out,
                        hipStream_t st) {
  if (s.n_groups == 0) return hipSuccess;
  if (!step_limits_ok(s)) return hipErrorInvalidValue;
  if (!route_lds_ok(s)) {
    // more router logits than LDS holds: the split route (scores to the
    // workspace, then the selection) serves the router-only call
    if (mode != ROUTE_TOPK || !split_shape(s)) return hipErrorInvalidValue;
    SplitArgs a = split_args(s, t, w, ws);
    a.r.scores_out = scores_out;
    a.idx_out = s.beta > 0 ? idx_out : nullptr;
    return s.d == 128 ? split_route_d<128>(a, s.B * s.Hkv, scores_out != nullptr, st)
                      : split_route_d<64>(a, s.B * s.Hkv, scores_out != nullptr, st);
  }
  return s.d == 128 ? summary_d<128>(s, t, w, ws, mode, given, scores_out, idx_out, st)
                    : summary_d<64>(s, t, w, ws, mode, given, scores_out, idx_out, st);
}

template <int D, typename TT = TokTile>
hipError_t token_d(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                   const int32_t* idx, const uint16_t* kdense, hipStream_t st,
                   const QjlKeys* qk = nullptr) {
  TokArgs a = tok_args(s, t);
  a.idx = idx;
  a.part = s.n_groups > 0 ? reinterpret_cast<const float*>(ws + w.part_off) : nullptr;
  a.kdense = kdense;
  if (qk) {
    a.l1_sk = qk->l1_sk; a.l1_gam = qk->l1_gam; a.l3_sk = qk->l3_sk; a.l3_gam = qk->l3_gam;
    a.S = qk->S;
  }
  const size_t smem = token_smem(D, s, !std::is_same_v<TT, TokTile>);
  if (s.group_n == 16)
    hipLaunchKernelGGL((token_kernel<D, 16, TT>), dim3((unsigned)(s.B * s.Hkv)), dim3(kThreads),
                       smem, st, a);
  else
    hipLaunchKernelGGL((token_kernel<D, 8, TT>), dim3((unsigned)(s.B * s.Hkv)), dim3(kThreads),
                       smem, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                       const int32_t* idx, hipStream_t st) {
  if (!step_limits_ok(s) || (s.n_groups > 0 && !route_lds_ok(s))) return hipErrorInvalidValue;
  return s.d == 128 ? token_d<128>(s, t, w, ws, idx, nullptr, st)
                    : token_d<64>(s, t, w, ws, idx, nullptr, st);
}

hipError_t launch_attn_prerope(const StepShape& s, const StepTensors& t, const Workspace& w,
                               char* ws, const int32_t* idx, const uint16_t* kdense,
                               hipStream_t st) {
  if (!step_limits_ok(s) || (s.n_groups > 0 && !route_lds_ok(s)) || (s.beta > 0 && !kdense))
    return hipErrorInvalidValue;
  return s.d == 128 ? token_d<128, TokTileK>(s, t, w, ws, idx, kdense, st)
                    : token_d<64, TokTileK>(s, t, w, ws, idx, kdense, st);
}

hipError_t launch_attn_qjl(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                           const int32_t* idx, const QjlKeys& qk, hipStream_t st) {
  if (!step_limits_ok(s) || (s.n_groups > 0 && !route_lds_ok(s)) || t.l3_staged ||
      s.l1_stride || s.ng_stride || !qk.S || (s.n_l1 > 0 && (!qk.l1_sk || !qk.l1_gam)) ||
      (s.beta > 0 && (!qk.l3_sk || !qk.l3_gam)))
    return hipErrorInvalidValue;
  return s.d == 128 ? token_d<128, TokTileQ>(s, t, w, ws, idx, nullptr, st, &qk)
                    : token_d<64, TokTileQ>(s, t, w, ws, idx, nullptr, st, &qk);
}

template <int D, int N>
hipError_t step_dn(const StepShape& s, const StepTensors& t, int32_t* idx_out, hipStream_t st) {
  SumArgs ra = sum_args(s, t);
  ra.want_topk = 1;
  ra.want_partial = 1;
  ra.idx = idx_out;
  TokArgs ta = tok_args(s, t);
  const dim3 grid((unsigned)(s.B * s.Hkv));
  const size_t smem = step_smem(s);
  if (fused_waves(s) == kFusedWavesFew) {
    constexpr int NW = kFusedWavesFew;
    if (t.agg == HSQ_AGG_MAX)
      hipLaunchKernelGGL((step_kernel<D, N, false, NW>), grid, dim3(NW * 64), smem, st, ra, ta);
    else
      hipLaunchKernelGGL((step_kernel<D, N, true, NW>), grid, dim3(NW * 64), smem, st, ra, ta);
  } else {
    constexpr int NW = kFusedWaves;
    if (t.agg == HSQ_AGG_MAX)
      hipLaunchKernelGGL((step_kernel<D, N, false, NW>), grid, dim3(NW * 64), smem, st, ra, ta);
    else
      hipLaunchKernelGGL((step_kernel<D, N, true, NW>), grid, dim3(NW * 64), smem, st, ra, ta);
  }
  return hipGetLastError();
}

int step_fused_ok(const StepShape& s) {
  return s.n_groups > 0 && s.n_groups <= kFusedMaxGroups && step_limits_ok(s) &&
         step_smem(s) <= kMaxFusedLds;
}

hipError_t launch_step(const StepShape& s, const StepTensors& t, int32_t* idx_out,
                       hipStream_t st) {
  if (!step_fused_ok(s)) return hipErrorInvalidValue;
  if (s.d == 128)
    return s.group_n == 16 ? step_dn<128, 16>(s, t, idx_out, st) : step_dn<128, 8>(s, t, idx_out, st);
  return s.group_n == 16 ? step_dn<64, 16>(s, t, idx_out, st) : step_dn<64, 8>(s, t, idx_out, st);
}

}  // namespace hsq
