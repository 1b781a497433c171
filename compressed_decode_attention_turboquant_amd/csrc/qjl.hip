// TQ-QKV key path for gfx950: TurboQuant key codes plus a 1-bit QJL sketch of
// the key's residual, and the corrected logits.
//
// [Ablation, Statistical Inference, and Validation for KV-Cache Compression,
// technical summary, "Experimental setup": TurboQuant may add a 1-bit
// Johnson-Lindenstrauss (QJL) residual sketch on the key or value path;
// "Key contributions" 1: TQ-QKV adds it on the key path.]  The estimator is
// the published QJL one (Zandieh, Daliri and Han, 2024): with S of i.i.d.
// N(0, 1) entries (m = d rows), sign(S u) and ||u|| give
// sqrt(pi/2) / m * ||u|| * <S z, sign(S u)> as an unbiased estimate of
// <z, u>.  Here u = y - c[code] is the TurboQuant error of the key in the
// rotated unit domain (y = R x / r), so for a query q the residual's share of
// the logit is r <R q, u>, estimated with z = R q; gamma = r ||u|| is stored.
//
// qjl_encode_kernel: one vector per d/8 lanes (as the codec's encoder) for
// the norm, rotation, threshold count and packing; then the pass's residuals
// go to LDS, and the projections S u of the whole pass are one small matrix
// product on fp32 MFMA against S, which sits in LDS for the work-group's loop
// over the vectors.  One rotation (one S) per launch.
// qjl_logits_kernel: S staged in LDS, R q and S R q for up to 8 query rows
// there too, then one key per d/8 lanes:
// r <R q, c[code]> + sqrt(pi/2)/m gamma <S R q, 1 - 2 bits>.
#include "encode_device.h"

namespace hsq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQWG = 256;

// LDS rows of S and of the residuals padded to d + 1 floats: the 16 (or 8)
// rows one vector's lanes read at a time, and the residual rows of different
// vectors, then fall in different banks.
template <int D>
constexpr int kSP = D + 1;

// S (d x d fp32, row-major) into LDS rows padded to d + 1 floats: coalesced
// loads, 16 in flight per thread before their LDS writes.
template <int D>
__device__ __forceinline__ void stage_S(float* s_S, const float* S, int tid) {
  constexpr int PER = D * D / kQWG;  // elements per thread
  constexpr int BATCH = 16;
  static_assert(PER % BATCH == 0, "whole batches");
#pragma unroll
  for (int b0 = 0; b0 < PER; b0 += BATCH) {
    float t[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) t[k] = S[(b0 + k) * kQWG + tid];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int e = (b0 + k) * kQWG + tid;
      s_S[(e / D) * kSP<D> + e % D] = t[k];
    }
  }
}

template <int D, int BITS, int DT>
__global__ __launch_bounds__(kQWG) void qjl_encode_kernel(QjlJob j) {
  constexpr int LPV = D / 8;
  constexpr int VPP = kQWG / LPV;  // vectors per pass
  constexpr int L = 1 << BITS;
  constexpr int NPOS = L / 2 - 1;
  constexpr int CB = D * BITS / 8;
  __shared__ float s_S[D * kSP<D>];
  __shared__ float s_u[VPP * kSP<D>];
  __shared__ float s_c[16];
  __shared__ int64_t s_out[VPP];  // output row of each vector of the pass
  const int tid = threadIdx.x, sub = tid % LPV, vl = tid / LPV;
  stage_S<D>(s_S, j.S, tid);
  if (tid < L) s_c[tid] = j.centroids[tid];
  uint32_t tpos[NPOS];
#pragma unroll
  for (int h = 0; h < NPOS; ++h) tpos[h] = __float_as_uint(j.thr[L / 2 + h]);
  const uint32_t sbyte = (j.signs[sub / 4] >> (8 * (sub % 4))) & 0xffu;
  __syncthreads();

  const int64_t passes = (j.n_vec + VPP - 1) / VPP;
  for (int64_t p = blockIdx.x; p < passes; p += gridDim.x) {
    const int64_t i = p * VPP + vl;
    const bool valid = i < j.n_vec;
    // input row and output row of this vector (gathered in a tier build)
    int64_t xr = i, orow = i;
    if (j.pos && valid) {
      const int64_t sq = i / j.per_seq;
      xr = j.x_base + sq * j.x_seq + j.pos[i];
      orow = j.out_base + sq * j.out_seq + (i - sq * j.per_seq);
    }
    if (sub == 0) s_out[vl] = orow;
    float v[8];
    if (valid) {
      load8<DT>(j.x, xr * D + 8 * sub, v);
    } else {
#pragma unroll
      for (int a = 0; a < 8; ++a) v[a] = 0.f;
    }
    // norm, rotation, threshold count and packing: the codec's arithmetic
    float ss = 0.f;
#pragma unroll
    for (int a = 0; a < 8; ++a) ss = fmaf(v[a], v[a], ss);
    float r, inv;
    norm_scale<D, true>(ss, r, inv);
#pragma unroll
    for (int a = 0; a < 8; ++a)
      v[a] = __uint_as_float(__float_as_uint(v[a]) ^ (((sbyte >> a) & 1u) << 31));
    fwht8xlanes<LPV>(v, sub);
    uint32_t packed = 0;
    float uu = 0.f;
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
      const float u = (r > 0.f) ? y - s_c[code] : 0.f;
      uu = fmaf(u, u, uu);
      s_u[vl * kSP<D> + 8 * sub + a] = u;
    }
    uu = lanes_sum<LPV>(uu);
    const bool wc = valid && j.codes != nullptr;  // codes and norms wanted
    uint8_t* crow = j.codes + (wc ? i : 0) * CB;
    if constexpr (BITS == 4) {
      if (wc) reinterpret_cast<uint32_t*>(crow)[sub] = packed;
    } else {
      const uint32_t nxt = __shfl_down(packed, 1, 64);
      const int qd = sub & 3;
      if (wc && qd < 3)
        reinterpret_cast<uint32_t*>(crow)[3 * (sub >> 2) + qd] =
            (packed >> (8 * qd)) | (nxt << (24 - 8 * qd));
    }
    if (valid && sub == 0) {
      if (wc) j.norms[i] = r;
      j.gamma[orow] = r * sqrtf(uu);
    }
    __syncthreads();
    // projections of the pass's residuals, P = U S^T (VPP x d), on fp32 MFMA
    // (16 x 16 x 4 blocks): the 8 output tiles of 16 x 16 go two to a wave.
    // In a tile, lane l holds P[4 (l / 16) + e][l % 16] (e < 4), so one
    // ballot per e gives, for the four vectors of each 16-lane row, 16
    // consecutive sketch bits.
    const int lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    constexpr int CT = D / 16;  // column tiles
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tile = 2 * wv + tt, rt = tile / CT, ct = tile % CT;
      const float* ua = s_u + (16 * rt + lr) * kSP<D> + lk;
      const float* sb = s_S + (16 * ct + lr) * kSP<D> + lk;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int k0 = 0; k0 < D; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ua[k0], sb[k0], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t b = __builtin_amdgcn_ballot_w64(acc[e] < 0.f);
        const int vv = 16 * rt + 4 * lk + e;  // vector of the pass
        const int64_t vi = p * VPP + vv;
        if (lr == 0 && vi < j.n_vec)
          *reinterpret_cast<uint16_t*>(j.sketch + s_out[vv] * (D / 8) + 2 * ct) =
              (uint16_t)(b >> (16 * lk));
      }
    }
    __syncthreads();
  }
}

template <int D, int BITS>
__global__ __launch_bounds__(kQWG) void qjl_logits_kernel(QjlLogitsJob j) {
  constexpr int LPV = D / 8;
  constexpr int CB = D * BITS / 8;
  __shared__ float s_qr[8 * D];  // R q per row
  __shared__ float s_sq[8 * D];  // S R q per row
  __shared__ float s_S[D * kSP<D>];
  __shared__ float s_c[16];
  const int tid = threadIdx.x;
  if (tid < (1 << BITS)) s_c[tid] = j.centroids[tid];
  stage_S<D>(s_S, j.S, tid);
  // R q = H D q / sqrt(d) for each query row (8 rows of LPV lanes)
  if (tid < 8 * LPV) {
    const int h = tid / LPV, sub = tid % LPV;
    float v[8];
    const uint32_t sb = (j.signs[sub / 4] >> (8 * (sub % 4))) & 0xffu;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const float x = (h < j.n_q) ? j.q[h * D + 8 * sub + a] : 0.f;
      v[a] = __uint_as_float(__float_as_uint(x) ^ (((sb >> a) & 1u) << 31));
    }
    fwht8xlanes<LPV>(v, sub);
#pragma unroll
    for (int a = 0; a < 8; ++a) s_qr[h * D + 8 * sub + a] = v[a] * rsqrtf((float)D);
  }
  __syncthreads();
  // consecutive threads take consecutive rows of S: padded LDS rows keep
  // their column reads on different banks
  for (int e = tid; e < j.n_q * D; e += kQWG) {
    const int h = e / D, row = e % D;
    float acc = 0.f;
#pragma unroll 16
    for (int i = 0; i < D; ++i) acc = fmaf(s_S[row * kSP<D> + i], s_qr[h * D + i], acc);
    s_sq[e] = acc;
  }
  __syncthreads();
  // one key per LPV lanes, 8 coordinates per lane (as the codec): each lane
  // forms its share of every row's two sums, then the LPV lanes add them
  const int sub = tid % LPV, kl = tid / LPV;
  constexpr int KPP = kQWG / LPV;  // keys per pass
  const float cq = 1.2533141373155003f / (float)D;  // sqrt(pi / 2) / m
  for (int64_t k0 = (int64_t)blockIdx.x * KPP; k0 < j.n_keys; k0 += (int64_t)gridDim.x * KPP) {
    const int64_t k = k0 + kl;
    const bool valid = k < j.n_keys;
    const int64_t kc = valid ? k : j.n_keys - 1;  // past the end: reread the last key
    const uint32_t* row = reinterpret_cast<const uint32_t*>(j.codes + kc * CB);
    uint32_t codes;
    if constexpr (BITS == 4) {
      codes = row[sub];
    } else {
      const int bit = 24 * sub, off = bit & 31;
      codes = row[bit >> 5] >> off;
      if (off > 8) codes |= row[(bit >> 5) + 1] << (32 - off);
      codes &= 0xffffffu;
    }
    const uint32_t sb = j.sketch[kc * (D / 8) + sub];
    const float r = j.norms[kc], g = j.gamma[kc];
    float c[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) c[a] = s_c[(codes >> (BITS * a)) & ((1u << BITS) - 1u)];
    for (int h = 0; h < j.n_q; ++h) {
      const f32x4* qv = reinterpret_cast<const f32x4*>(s_qr + h * D + 8 * sub);
      const f32x4* sv = reinterpret_cast<const f32x4*>(s_sq + h * D + 8 * sub);
      const f32x4 q0 = qv[0], q1 = qv[1], s0 = sv[0], s1 = sv[1];
      float dot = 0.f, corr = 0.f;
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const float qa = a < 4 ? q0[a] : q1[a - 4];
        const float sa = a < 4 ? s0[a] : s1[a - 4];
        dot = fmaf(qa, c[a], dot);
        corr += ((sb >> a) & 1u) ? -sa : sa;
      }
      dot = lanes_sum<LPV>(dot);
      corr = lanes_sum<LPV>(corr);
      if (valid && sub == 0) j.out[h * j.n_keys + k] = j.scale * (r * dot + cq * g * corr);
    }
  }
}

template <int D, int BITS>
hipError_t qjl_encode_db(const QjlJob& j, hipStream_t s) {
  constexpr int VPP = kQWG / (D / 8);
  const int64_t passes = (j.n_vec + VPP - 1) / VPP;
  // two work-groups fit a CU's LDS (S and the residuals, 74 KB each): one
  // resident round of 512 stages S once each and strides over the passes
  const unsigned grid = (unsigned)(passes < 512 ? passes : 512);
  if (j.dtype == HSQ_F32)
    hipLaunchKernelGGL((qjl_encode_kernel<D, BITS, HSQ_F32>), dim3(grid), dim3(kQWG), 0, s, j);
  else
    hipLaunchKernelGGL((qjl_encode_kernel<D, BITS, HSQ_BF16>), dim3(grid), dim3(kQWG), 0, s, j);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t qjl_logits_db(const QjlLogitsJob& j, hipStream_t s) {
  // every work-group forms R q and S R q once, then loops over its keys
  constexpr int KPP = kQWG / (D / 8);
  const int64_t passes = (j.n_keys + KPP - 1) / KPP;
  const int64_t grid = passes < 512 ? passes : 512;
  hipLaunchKernelGGL((qjl_logits_kernel<D, BITS>), dim3((unsigned)grid), dim3(kQWG), 0, s, j);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qjl_encode(const QjlJob& j, hipStream_t s) {
  if (j.n_vec <= 0) return hipSuccess;
  if (j.d == 128) return j.bits == 4 ? qjl_encode_db<128, 4>(j, s) : qjl_encode_db<128, 3>(j, s);
  return j.bits == 4 ? qjl_encode_db<64, 4>(j, s) : qjl_encode_db<64, 3>(j, s);
}

hipError_t launch_qjl_logits(const QjlLogitsJob& j, hipStream_t s) {
  if (j.n_keys <= 0 || j.n_q <= 0) return hipSuccess;
  if (j.d == 128) return j.bits == 4 ? qjl_logits_db<128, 4>(j, s) : qjl_logits_db<128, 3>(j, s);
  return j.bits == 4 ? qjl_logits_db<64, 4>(j, s) : qjl_logits_db<64, 3>(j, s);
}

}  // namespace hsq
