// Gather of fetched L3 records into an HBM staging buffer.
//
// [Tamarin (HSQ) summary, section 2, "Decode process", step 2: the originals
// of the selected groups are fetched from the CPU-RAM archive.]  The archive
// is pinned, mapped host memory; the kernel reads it through its device
// alias, so the transfer crosses PCIe while the group indices stay on the
// device.
//
// A work-group moves kRecs records (consecutive selection slots).  It reads
// their indices once, then its 256 lanes sweep the records' 16-byte words in
// order, kUnroll loads in flight per lane, so every PCIe read request is a
// whole aligned run.  The launch is deliberately narrow: a PCIe read holds
// its CU's memory path for microseconds, and kernels whose work-groups share
// a CU with a gather work-group (the route and attend launches of another
// micro-batch) slow down with it.  128 records per work-group with two loads
// in flight per lane keeps the link near a pinned copy's rate on a few CUs.
//
// Ordered form (turn != null): gathers issued on different streams take the
// link in turn without host-side events.  Each work-group first waits until
// *turn reaches `after` (thread 0 polls with an agent-scope atomic load,
// sleeping between polls, for at most kTurnWaitTicks of the 100 MHz real-time
// clock, then goes ahead regardless: the wait orders the link, never the
// data), and adds its record count to *turn once all its loads have landed.
#include "hsq_internal.h"

namespace hsq {
namespace {

constexpr int kRecs = 128;
constexpr int kUnroll = 2;
constexpr int kGatherThreads = 256;
constexpr uint32_t kDrop = 0x80000000u;  // buffer offset past any range: the store is dropped
constexpr uint64_t kTurnWaitTicks = 200000;  // 2 ms at 100 MHz: longest wait for the turn

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const uint8_t* __restrict__ src, size_t rec_bytes, int n_groups,
    const int32_t* __restrict__ idx, int beta, int64_t n_slots, uint8_t* __restrict__ dst,
    uint32_t* turn, uint32_t after) {
  __shared__ int64_t s_off[kRecs];  // byte offset of each record in src, -1 if invalid
  const int tid = threadIdx.x;
  const int64_t s0 = (int64_t)blockIdx.x * kRecs;
  const int n16 = (int)(rec_bytes / 16);
  const int nrec = (int)min<int64_t>(kRecs, n_slots - s0);
  if (turn != nullptr && tid == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((int32_t)(__hip_atomic_load(turn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                     after) < 0 &&
           __builtin_amdgcn_s_memrealtime() - t0 < kTurnWaitTicks)
      __builtin_amdgcn_s_sleep(4);
  }
  if (tid < nrec) {
    const int64_t slot = s0 + tid;  // unit * beta + i
    const int g = idx[slot];
    s_off[tid] = (g >= 0 && g < n_groups) ? ((slot / beta) * n_groups + g) * (int64_t)rec_bytes
                                          : -1;  // invalid selection: staging left untouched
  }
  __syncthreads();
  const int total = nrec * n16;
  const uint4* sw = reinterpret_cast<const uint4*>(src);
  // this work-group's staging records; stores at kDrop fall outside the
  // range and are dropped, so invalid records and the sweep's tail need no
  // branch (a branch would hold each load back to its store)
  const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
      dst + s0 * (int64_t)rec_bytes, 0, (int)(nrec * rec_bytes), 0x00020000);
  for (int k0 = tid; k0 < total; k0 += kUnroll * kGatherThreads) {
    uint4 v[kUnroll];
    uint32_t so[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      // a lane with no word loads the first word of src and drops it
      const int k = k0 + j * kGatherThreads;
      const int r = k < total ? k / n16 : 0;
      const int64_t off = s_off[r];
      const bool ok = off >= 0 && k < total;
      v[j] = sw[ok ? off / 16 + (k - r * n16) : 0];
      so[j] = ok ? 16u * (uint32_t)k : kDrop;
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      __builtin_amdgcn_raw_buffer_store_b128((u32x4){v[j].x, v[j].y, v[j].z, v[j].w}, dr,
                                             (int)so[j], 0, 0);
  }
  if (turn != nullptr) {
    __syncthreads();  // every lane's loads have returned (its stores consumed them)
    if (tid == 0)
      __hip_atomic_fetch_add(turn, (uint32_t)nrec, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_gather(const uint8_t* src, size_t rec_bytes, int units, int n_groups,
                         const int32_t* idx, int beta, uint8_t* dst, uint32_t* turn,
                         uint32_t after, hipStream_t st) {
  const int64_t n_slots = (int64_t)units * beta;
  if (n_slots <= 0) return hipSuccess;
  // one work-group's staging range is a 32-bit buffer range
  if ((int64_t)kRecs * (int64_t)rec_bytes >= (int64_t)kDrop) return hipErrorInvalidValue;
  const int64_t blocks = (n_slots + kRecs - 1) / kRecs;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(kGatherThreads), 0, st, src,
                     rec_bytes, n_groups, idx, beta, n_slots, dst, turn, after);
  return hipGetLastError();
}

}  // namespace hsq
