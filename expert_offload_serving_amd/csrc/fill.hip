// Expert copies: cache-miss fills from the pinned host pool (the pages fetch
// missing experts over PCIe on demand: aiforradalom.hu FreeToken article,
// section "A Mixture-of-Experts (MoE) kihívásai és a FreeToken
// megoldásai"), resize moves, and a plain copy used as a bandwidth probe.
//
// Fills run as a device kernel that reads the device-mapped pinned pool, so
// the miss list never leaves the GPU and the decode call needs no host sync.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Copy n records of `units` 16-byte units each; all threads stride over each
// record with 4 loads in flight.
__device__ __forceinline__ void copy_record(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                            size_t units) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < units; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < units; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void fill_kernel(const FillEntry* __restrict__ fills,
                                                   const DevMeta* __restrict__ meta, int max_fill,
                                                   size_t units) {
  const int n = min(meta->n_fill, max_fill);
  for (int r = 0; r < n; r++)
    copy_record(reinterpret_cast<const u32x4*>(fills[r].src), reinterpret_cast<u32x4*>(fills[r].dst),
                units);
}

__global__ __launch_bounds__(256) void copy_pairs_kernel(const FillEntry* __restrict__ pairs, int n,
                                                         size_t units) {
  for (int r = 0; r < n; r++)
    copy_record(reinterpret_cast<const u32x4*>(pairs[r].src), reinterpret_cast<u32x4*>(pairs[r].dst),
                units);
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, size_t units) {
  copy_record(src, dst, units);
}

constexpr int kCopyBlocks = 1024;
// Fills read mapped host memory at PCIe rate: a workgroup per CU keeps far
// more than enough in flight, and a launch with nothing to copy (every
// expert a hit) costs less to dispatch.
constexpr int kFillBlocks = 256;

}  // namespace

hipError_t launch_fill(const FillEntry* fills, const DevMeta* meta, int max_fill, size_t bytes,
                       hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (max_fill <= 0) return hipSuccess;
  MOE_LAUNCH(fill_kernel, kFillBlocks, 256, 0, st, ev0, ev1, fills, meta, max_fill, bytes / 16);
  return hipGetLastError();
}

hipError_t launch_copy_pairs(const FillEntry* pairs, int n, size_t bytes, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  copy_pairs_kernel<<<kCopyBlocks, 256, 0, st>>>(pairs, n, bytes / 16);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t n_bytes, hipStream_t st) {
  probe_copy_kernel<<<4096, 256, 0, st>>>(reinterpret_cast<const u32x4*>(src),
                                         reinterpret_cast<u32x4*>(dst), n_bytes / 16);
  return hipGetLastError();
}

}  // namespace moe
