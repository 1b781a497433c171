// Decode-time tier maintenance for gfx950: one appended token per unit, in
// one launch.
//
// [Tamarin (HSQ) summary, section 2, "Three-tier architecture": L1 holds the
// sinks, the recent window and the reader-marked tokens at 4 bits; the other
// tokens form groups of N with a 3-bit summary (L2) and 4-bit originals
// (L3).]  The tiers after an append are the ones the compress-time build
// gives for the longer context: the token leaving the window becomes a
// pending L1 token (the grouping remainder), and N pending tokens are sealed
// into the next group.
//
// One 64-lane work-group per unit, two phases around one barrier:
//   (A) moves, every lane: the window slot's codes, norm and raw vector go to
//       the next pending slot; on a seal the N pending tokens' codes and
//       norms form the group's L3 record [K codes][K norms][V codes][V norms]
//       (the last pending token is the window slot's, read where it is).
//   (B) encodes, one vector per d/8 lanes with the codec's encoder: the new
//       K and V at 4 bits into the window slot's L1 row (their raw vectors
//       into its raw row); on a seal the K and V summaries, the 3-bit code of
//       the mean of the N pending raw rows, summed in position order as the
//       compress-time build does, so both give the same bits.
// (B) writes only the window slot's rows and the new group's summaries; (A)
// reads the window slot's rows and writes the pending rows that (B) reads,
// so the barrier orders every cross-lane dependency.
#include "encode_device.h"

namespace hsq {
namespace {

template <int D, int DT>
__global__ __launch_bounds__(64) void append_kernel(AppendJob a, Div32 one) {
  constexpr int LPV = D / 8;                          // lanes per vector
  constexpr int CW = D / 8;                           // 32-bit words of 4-bit codes per row
  constexpr int RW = D * (DT == HSQ_F32 ? 4 : 2) / 4; // 32-bit words per raw row
  const int u = blockIdx.x, lane = threadIdx.x;
  const int kvh = u % a.Hkv;
  const size_t l1u = (size_t)u * a.l1_cap;
  const size_t src = l1u + a.n_fix + a.slot;          // the window slot's L1 row
  const size_t pend0 = l1u + a.n_fix + a.n_recent;
  const size_t dst = pend0 + a.pending;
  const size_t ru = (size_t)u * (a.n_recent + a.group_n);
  uint32_t* lk = reinterpret_cast<uint32_t*>(a.l1k);
  uint32_t* lv = reinterpret_cast<uint32_t*>(a.l1v);
  uint32_t* rk = static_cast<uint32_t*>(a.raw_k);
  uint32_t* rv = static_cast<uint32_t*>(a.raw_v);

  // (A) the window slot's token -> pending slot
  for (int w = lane; w < CW; w += 64) {
    lk[dst * CW + w] = lk[src * CW + w];
    lv[dst * CW + w] = lv[src * CW + w];
  }
  if (lane == 0) {
    a.l1k_n[dst] = a.l1k_n[src];
    a.l1v_n[dst] = a.l1v_n[src];
  }
  const size_t rslot = (ru + a.slot) * RW, rpend = (ru + a.n_recent + a.pending) * RW;
  for (int w = lane; w < RW; w += 64) {
    rk[rpend + w] = rk[rslot + w];
    rv[rpend + w] = rv[rslot + w];
  }
  if (a.seal) {
    const int N = a.group_n;
    uint32_t* rec = reinterpret_cast<uint32_t*>(a.l3) +
                    ((size_t)u * a.ng_cap + a.ng) * ((size_t)N * (D + 8) / 4);
    uint32_t* rec_kn = rec + N * CW;
    uint32_t* rec_v = rec_kn + N;
    uint32_t* rec_vn = rec_v + N * CW;
    for (int e = lane; e < N * CW; e += 64) {
      const int r = e / CW, w = e - r * CW;
      const size_t row = (r == a.pending) ? src : pend0 + r;
      rec[e] = lk[row * CW + w];
      rec_v[e] = lv[row * CW + w];
    }
    for (int r = lane; r < N; r += 64) {
      const size_t row = (r == a.pending) ? src : pend0 + r;
      rec_kn[r] = __float_as_uint(a.l1k_n[row]);
      rec_vn[r] = __float_as_uint(a.l1v_n[row]);
    }
  }
  __syncthreads();

  // (B) lane groups: 0 = new K, 1 = new V (4-bit); on a seal 2 = K summary,
  // 3 = V summary (3-bit)
  const int grp = lane / LPV, sub = lane % LPV;
  EncodeDivs q{};
  q.rec = one;
  EncodeJob j{};
  j.n_vec = 1;
  if (grp < 2) {
    const bool isv = grp == 1;
    const void* x = isv ? a.v_new : a.k_new;
    const uint32_t* nw = static_cast<const uint32_t*>(x) + (size_t)u * RW;
    uint32_t* rr = (isv ? rv : rk) + rslot;
    for (int w = sub; w < RW; w += LPV) rr[w] = nw[w];
    float v[8];
    load8<DT>(x, (int64_t)u * D + 8 * sub, v);
    const uint32_t sword = (isv ? a.v_signs : a.k_signs)[kvh * (D / 32) + sub / 4];
    uint32_t tpos[7];
#pragma unroll
    for (int h = 0; h < 7; ++h) tpos[h] = __float_as_uint(a.thr4[8 + h]);
    j.group_n = 1;
    j.codes = (isv ? a.l1v : a.l1k) + (l1u + a.n_fix + a.slot) * (D / 2);
    j.norms = (isv ? a.l1v_n : a.l1k_n) + l1u + a.n_fix + a.slot;
    encode_one<D, 4, true>(j, q, 0u, sub, v, sword, tpos, false, nullptr);
  } else if (grp < 4 && a.seal) {
    const bool isv = grp == 3;
    const void* x = isv ? a.raw_v : a.raw_k;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < a.group_n; ++k) {
      float t[8];
      load8<DT>(x, (int64_t)(ru + a.n_recent + k) * D + 8 * sub, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += t[e];
    }
    const uint32_t sword = (isv ? a.v_signs : a.k_signs)[kvh * (D / 32) + sub / 4];
    uint32_t tpos[3];
#pragma unroll
    for (int h = 0; h < 3; ++h) tpos[h] = __float_as_uint(a.thr3[4 + h]);
    j.group_n = a.group_n;
    j.codes = (isv ? a.l2v : a.l2k) + ((size_t)u * a.ng_cap + a.ng) * (3 * D / 8);
    j.norms = (isv ? a.l2v_n : a.l2k_n) + (size_t)u * a.ng_cap + a.ng;
    encode_one<D, 3, true>(j, q, 0u, sub, v, sword, tpos, false, nullptr);
  }
}

template <int D>
hipError_t append_d(const AppendJob& j, hipStream_t s) {
  const Div32 one = make_div32(1);
  if (j.dtype == HSQ_F32)
    hipLaunchKernelGGL((append_kernel<D, HSQ_F32>), dim3((unsigned)j.units), dim3(64), 0, s, j, one);
  else
    hipLaunchKernelGGL((append_kernel<D, HSQ_BF16>), dim3((unsigned)j.units), dim3(64), 0, s, j, one);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_append(const AppendJob& j, hipStream_t s) {
  if (j.units <= 0) return hipSuccess;
  return j.d == 128 ? append_d<128>(j, s) : append_d<64>(j, s);
}

}  // namespace hsq
