// Decode-time tier maintenance for gfx950: the data moves of one appended
// token per unit.
//
// [Tamarin (HSQ) summary, section 2, "Three-tier architecture": L1 holds the
// sinks, the recent window and the reader-marked tokens; the other tokens
// form groups of N with a 3-bit summary (L2) and 4-bit originals (L3).]  The
// tiers after an append are the ones the compress-time build gives for the
// longer context: the token leaving the window becomes a pending L1 token
// (the grouping remainder), and N pending tokens are sealed into the next
// group.  The encodes of that step (the new token at 4 bits, the summaries
// of a sealed group at 3 bits) run in the codec kernels; this kernel does the
// moves around them:
//   * the window slot's codes and norm -> the next pending L1 row, and its raw
//     vector -> the next pending raw row (the raw vectors of the window and of
//     the pending tokens are kept for the group-mean summaries);
//   * the new token's raw vector -> the window slot's raw row;
//   * on a seal, the N pending tokens' codes and norms -> the group's L3
//     record [K codes][K norms][V codes][V norms].  The last pending token is
//     the one this call moves, so its row is read from the window slot, which
//     this launch does not write: no thread reads what another writes, and
//     the work-group needs no barrier.
// One 64-lane work-group per unit; every access is a 32-bit word.
#include "hsq_internal.h"

namespace hsq {
namespace {

__global__ __launch_bounds__(64) void evict_kernel(EvictJob j) {
  const int u = blockIdx.x, tid = threadIdx.x;
  const int cw = j.d / 8;  // 32-bit words of 4-bit codes per row
  const size_t l1u = (size_t)u * j.l1_cap;
  const size_t src = l1u + j.n_fix + j.slot;
  const size_t pend0 = l1u + j.n_fix + j.n_recent;
  const size_t dst = pend0 + j.pending;
  uint32_t* lk = reinterpret_cast<uint32_t*>(j.l1k);
  uint32_t* lv = reinterpret_cast<uint32_t*>(j.l1v);
  for (int w = tid; w < cw; w += 64) {
    lk[dst * cw + w] = lk[src * cw + w];
    lv[dst * cw + w] = lv[src * cw + w];
  }
  if (tid == 0) {
    j.l1k_n[dst] = j.l1k_n[src];
    j.l1v_n[dst] = j.l1v_n[src];
  }

  const int rw = j.d * j.esize / 4;  // words per raw row
  const size_t ru = (size_t)u * (j.n_recent + j.group_n);
  uint32_t* rk = static_cast<uint32_t*>(j.raw_k);
  uint32_t* rv = static_cast<uint32_t*>(j.raw_v);
  const uint32_t* nk = static_cast<const uint32_t*>(j.k_new) + (size_t)u * rw;
  const uint32_t* nv = static_cast<const uint32_t*>(j.v_new) + (size_t)u * rw;
  const size_t rslot = (ru + j.slot) * rw, rpend = (ru + j.n_recent + j.pending) * rw;
  for (int w = tid; w < rw; w += 64) {
    const uint32_t ok = rk[rslot + w], ov = rv[rslot + w];
    rk[rpend + w] = ok;
    rv[rpend + w] = ov;
    rk[rslot + w] = nk[w];
    rv[rslot + w] = nv[w];
  }
  if (!j.seal) return;

  const int N = j.group_n;
  const size_t recw = (size_t)N * (j.d + 8) / 4;  // words per record
  uint32_t* rec = reinterpret_cast<uint32_t*>(j.l3) + ((size_t)u * j.ng_cap + j.ng) * recw;
  uint32_t* rec_kn = rec + N * cw;
  uint32_t* rec_v = rec_kn + N;
  uint32_t* rec_vn = rec_v + N * cw;
  for (int e = tid; e < N * cw; e += 64) {
    const int r = e / cw, w = e - r * cw;
    const size_t row = (r == j.pending) ? src : pend0 + r;
    rec[e] = lk[row * cw + w];
    rec_v[e] = lv[row * cw + w];
  }
  for (int r = tid; r < N; r += 64) {
    const size_t row = (r == j.pending) ? src : pend0 + r;
    rec_kn[r] = __float_as_uint(j.l1k_n[row]);
    rec_vn[r] = __float_as_uint(j.l1v_n[row]);
  }
}

}  // namespace

hipError_t launch_cache_evict(const EvictJob& j, hipStream_t s) {
  if (j.units <= 0) return hipSuccess;
  hipLaunchKernelGGL(evict_kernel, dim3((unsigned)j.units), dim3(64), 0, s, j);
  return hipGetLastError();
}

}  // namespace hsq
