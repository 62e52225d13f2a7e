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

// Device-to-device copy of `units` 16-byte units (resize moves, the copy
// probe): a workgroup takes contiguous chunks of 8 x 256 units (32 KB), each
// thread 8 units of a chunk in flight; loads and stores are nontemporal, since
// neither side is read again soon.
constexpr int kD2dThreads = 256, kD2dDepth = 8;
__device__ __forceinline__ void copy_d2d(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                         size_t units) {
  constexpr size_t kChunk = (size_t)kD2dThreads * kD2dDepth;
  const size_t n_chunks = units / kChunk;
  for (size_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const size_t base = c * kChunk + threadIdx.x;
    u32x4 v[kD2dDepth];
#pragma unroll
    for (int i = 0; i < kD2dDepth; i++) v[i] = __builtin_nontemporal_load(src + base + i * kD2dThreads);
#pragma unroll
    for (int i = 0; i < kD2dDepth; i++) __builtin_nontemporal_store(v[i], dst + base + i * kD2dThreads);
  }
  // the tail (fewer than a chunk's units), one unit per thread of the grid
  for (size_t i = n_chunks * kChunk + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < units;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// A confined fill (one that runs beside expert kernels) has workgroups that
// each take (nearly) a whole CU's LDS, so that no expert-kernel workgroup
// (all of them use LDS) is placed beside them: a workgroup sharing a CU with
// reads of mapped host memory waits behind them in the CU's memory
// pipeline, and a kernel running beside the fill would finish only when the
// fill does.
constexpr int kFillHoldBytes = 161792;

template <bool Confined>
__global__ __launch_bounds__(1024) void fill_kernel(const FillEntry* __restrict__ fills,
                                                    const DevMeta* __restrict__ meta, int max_fill,
                                                    size_t units) {
  if constexpr (Confined) {
    __shared__ uint8_t hold[kFillHoldBytes];
    volatile uint8_t* held = hold;
    held[threadIdx.x] = 0;  // keeps the allocation
  }
  const int n = min(meta->n_fill, max_fill);
  for (int r = 0; r < n; r++)
    copy_record(reinterpret_cast<const u32x4*>(fills[r].src), reinterpret_cast<u32x4*>(fills[r].dst),
                units);
}
__global__ __launch_bounds__(kD2dThreads) void copy_pairs_kernel(const FillEntry* __restrict__ pairs,
                                                                  int n, size_t units) {
  for (int r = 0; r < n; r++)
    copy_d2d(reinterpret_cast<const u32x4*>(pairs[r].src), reinterpret_cast<u32x4*>(pairs[r].dst),
             units);
}

__global__ __launch_bounds__(kD2dThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst, size_t units) {
  copy_d2d(src, dst, units);
}

constexpr int kCopyBlocks = 1024;
// Fills read mapped host memory at PCIe rate (about 56 GB/s).  Alone, a
// workgroup of 256 on every CU keeps enough in flight and costs little to
// dispatch when there is nothing to copy.  Confined, eight workgroups of
// 1024 (one CU per XCD) still copy a 20 MB record at 55.7 GB/s, and an
// HBM-streaming kernel beside them runs at 26 us instead of 22 us alone
// (356 us when its workgroups may share the copy's CUs).
constexpr int kFillBlocks = 256, kFillThreads = 256;
constexpr int kConfinedFillBlocks = 8, kConfinedFillThreads = 1024;
}  // namespace
hipError_t launch_fill(const FillEntry* fills, const DevMeta* meta, int max_fill, size_t bytes,
                       bool confined, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (max_fill <= 0) return hipSuccess;
  if (confined)
    MOE_LAUNCH(fill_kernel<true>, kConfinedFillBlocks, kConfinedFillThreads, 0, st, ev0, ev1,
               fills, meta, max_fill, bytes / 16);
  else
    MOE_LAUNCH(fill_kernel<false>, kFillBlocks, kFillThreads, 0, st, ev0, ev1, fills, meta,
               max_fill, bytes / 16);
  return hipGetLastError();
}
hipError_t launch_copy_pairs(const FillEntry* pairs, int n, size_t bytes, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  copy_pairs_kernel<<<kCopyBlocks, kD2dThreads, 0, st>>>(pairs, n, bytes / 16);
  return hipGetLastError();
}

// One thread stores `seq` to a word of pinned host memory with a
// system-scope release (a vector store), after the work queued before it on
// the stream: the host reads it to learn that work is done without a HIP
// call.
__global__ void signal_kernel(uint64_t* flag, uint64_t seq) {
  __hip_atomic_store(flag, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_signal(uint64_t* host_flag, uint64_t seq, hipStream_t st) {
  signal_kernel<<<1, 1, 0, st>>>(host_flag, seq);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t n_bytes, hipStream_t st) {
  probe_copy_kernel<<<kCopyBlocks, kD2dThreads, 0, st>>>(reinterpret_cast<const u32x4*>(src),
                                         reinterpret_cast<u32x4*>(dst), n_bytes / 16);
  return hipGetLastError();
}

}  // namespace moe
