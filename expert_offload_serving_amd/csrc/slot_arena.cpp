// Memory of the HBM expert-cache slots: one device address range reserved
// for the largest capacity, backed by physical chunks that are mapped and
// unmapped as the capacity changes.  Slot s always lives at base + s*stride,
// so a resize moves only the records that change slots, and shrinking
// returns the memory past the new capacity without touching the rest (the
// pages let the cache budget change at run time without a restart:
// aipolix.com FreeToken article, sixth paragraph).
#include <algorithm>

#include "moe_internal.h"

namespace moe {

namespace {

hipMemAllocationProp chunk_prop(int device) {
  hipMemAllocationProp p = {};
  p.type = hipMemAllocationTypePinned;
  p.location.type = hipMemLocationTypeDevice;
  p.location.id = device;
  return p;
}

// Map chunk i (creating its physical memory); on failure nothing of it stays.
hipError_t map_chunk(SlotArena& a, size_t i, hipMemGenericAllocationHandle_t* out) {
  const hipMemAllocationProp prop = chunk_prop(a.device);
  hipMemGenericAllocationHandle_t h;
  hipError_t e = hipMemCreate(&h, a.chunk, &prop, 0);
  if (e != hipSuccess) return e;
  uint8_t* at = a.base + i * a.chunk;
  e = hipMemMap(at, a.chunk, 0, h, 0);
  if (e != hipSuccess) {
    (void)hipMemRelease(h);
    return e;
  }
  hipMemAccessDesc acc = {};
  acc.location = prop.location;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  e = hipMemSetAccess(at, a.chunk, &acc, 1);
  if (e != hipSuccess) {
    (void)hipMemUnmap(at, a.chunk);
    (void)hipMemRelease(h);
    return e;
  }
  *out = h;
  return hipSuccess;
}

void unmap_chunk(SlotArena& a, size_t i) {
  (void)hipMemUnmap(a.base + i * a.chunk, a.chunk);
  (void)hipMemRelease(a.chunks[i]);
}

}  // namespace

hipError_t arena_init(SlotArena& a, int device, size_t max_bytes) {
  a.device = device;
  // About 32 chunks for the largest capacity, a power of two between 64 MiB
  // and 1 GiB: unmapping and releasing a chunk costs about 0.27 ms whatever
  // its size (measured on MI355X), so a shrink of a GLM-sized cache from 1228
  // to 614 slots releases about 11 chunks rather than hundreds, while a small
  // cache keeps at most 64 MiB past its last slot.
  a.chunk = kSlotChunkMin;
  while (a.chunk < kSlotChunkMax && a.chunk * 32 < max_bytes) a.chunk *= 2;
  const hipMemAllocationProp prop = chunk_prop(device);
  size_t gran = 0;
  hipError_t e = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum);
  if (e != hipSuccess) return e;
  if (gran == 0 || a.chunk % gran) return hipErrorNotSupported;
  a.reserved = std::max<size_t>((max_bytes + a.chunk - 1) / a.chunk, 1) * a.chunk;
  void* p = nullptr;
  // chunk-aligned, so that every chunk can use the largest page size
  e = hipMemAddressReserve(&p, a.reserved, a.chunk, nullptr, 0);
  if (e != hipSuccess) {
    a.reserved = 0;
    return e;
  }
  a.base = static_cast<uint8_t*>(p);
  return hipSuccess;
}

hipError_t arena_ensure(SlotArena& a, size_t bytes) {
  const size_t need = (bytes + a.chunk - 1) / a.chunk;
  if (need * a.chunk > a.reserved) return hipErrorInvalidValue;
  const size_t had = a.chunks.size();
  for (size_t i = had; i < need; i++) {
    hipMemGenericAllocationHandle_t h;
    const hipError_t e = map_chunk(a, i, &h);
    if (e != hipSuccess) {
      arena_trim(a, had * a.chunk);  // all or nothing
      return e;
    }
    a.chunks.push_back(h);
  }
  return hipSuccess;
}

void arena_trim(SlotArena& a, size_t bytes) {
  const size_t keep = (bytes + a.chunk - 1) / a.chunk;
  while (a.chunks.size() > keep) {
    unmap_chunk(a, a.chunks.size() - 1);
    a.chunks.pop_back();
  }
}

void arena_free(SlotArena& a) {
  if (!a.base) return;
  arena_trim(a, 0);
  (void)hipMemAddressFree(a.base, a.reserved);
  a.base = nullptr;
  a.reserved = 0;
}

}  // namespace moe
