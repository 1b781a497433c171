// Gather of fetched L3 records into an HBM staging buffer.
//
// [Tamarin (HSQ) summary, section 2, "Decode process", step 2: the originals
// of the selected groups are fetched from the CPU-RAM archive.]  The archive
// is pinned, mapped host memory; the kernel reads it through its device
// alias, so the transfer crosses PCIe while the group indices stay on the
// device.  A work-group moves kRecs records (consecutive selection slots):
// its 256 lanes sweep their 16-byte words in order, so every PCIe read
// request is a whole aligned run and a launch has few, long-lived
// work-groups (one record per work-group leaves most lanes of the last
// sweep idle and reaches only 90% of a same-size pinned copy).
#include "hsq_internal.h"

namespace hsq {
namespace {

constexpr int kRecs = 16;

__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ src, size_t rec_bytes,
                                                     int n_groups, const int32_t* __restrict__ idx,
                                                     int beta, int64_t n_slots,
                                                     uint8_t* __restrict__ dst) {
  const int64_t s0 = (int64_t)blockIdx.x * kRecs;
  const int n16 = (int)(rec_bytes / 16);
  const int nrec = (int)min<int64_t>(kRecs, n_slots - s0);
  for (int k = threadIdx.x; k < nrec * n16; k += blockDim.x) {
    const int r = k / n16, e = k - r * n16;
    const int64_t slot = s0 + r;             // unit * beta + i
    const int64_t unit = slot / beta;
    const int g = idx[slot];
    if (g < 0 || g >= n_groups) continue;   // invalid selection: leave staging untouched
    const uint4* s = reinterpret_cast<const uint4*>(src + (unit * n_groups + g) * rec_bytes);
    reinterpret_cast<uint4*>(dst + slot * rec_bytes)[e] = s[e];
  }
}

}  // namespace

hipError_t launch_gather(const uint8_t* src, size_t rec_bytes, int units, int n_groups,
                         const int32_t* idx, int beta, uint8_t* dst, hipStream_t st) {
  const int64_t n_slots = (int64_t)units * beta;
  if (n_slots <= 0) return hipSuccess;
  const int64_t blocks = (n_slots + kRecs - 1) / kRecs;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, rec_bytes,
                     n_groups, idx, beta, n_slots, dst);
  return hipGetLastError();
}

}  // namespace hsq
