// Gather of fetched L3 records into an HBM staging buffer.
//
// [Tamarin (HSQ) summary, section 2, "Decode process", step 2: the originals
// of the selected groups are fetched from the CPU-RAM archive.]  The archive
// is pinned, mapped host memory; the kernel reads it through its device
// alias, so the transfer crosses PCIe while the group indices stay on the
// device.  One work-group per (unit, fetched slot); 16-byte lanes, so a
// record of N*(d+8) bytes moves in ceil(rec/16/256) coalesced sweeps.
#include "hsq_internal.h"

namespace hsq {
namespace {

__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ src, size_t rec_bytes,
                                                     int n_groups, const int32_t* __restrict__ idx,
                                                     int beta, uint8_t* __restrict__ dst) {
  const int64_t slot = blockIdx.x;            // unit * beta + i
  const int64_t unit = slot / beta;
  const int g = idx[slot];
  if (g < 0 || g >= n_groups) return;         // invalid selection: leave staging untouched
  const uint4* s = reinterpret_cast<const uint4*>(src + (unit * n_groups + g) * rec_bytes);
  uint4* d = reinterpret_cast<uint4*>(dst + slot * rec_bytes);
  const int n16 = (int)(rec_bytes / 16);
  for (int k = threadIdx.x; k < n16; k += blockDim.x) d[k] = s[k];
}

}  // namespace

hipError_t launch_gather(const uint8_t* src, size_t rec_bytes, int units, int n_groups,
                         const int32_t* idx, int beta, uint8_t* dst, hipStream_t st) {
  const int64_t blocks = (int64_t)units * beta;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, rec_bytes,
                     n_groups, idx, beta, dst);
  return hipGetLastError();
}

}  // namespace hsq
