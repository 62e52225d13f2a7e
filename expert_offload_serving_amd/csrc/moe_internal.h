// Internal declarations of libmoe: context, device layouts, kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// MXFP4 expert record in the library's tiled layout.
//
// A matrix W [N rows][K] (rows = output features) is cut into atoms of
// 16 rows x 128 K (four MX blocks per row).  One atom is 1088 contiguous
// bytes, one lane of a wave per MX block:
//   bytes [16 l, 16 l + 16), l = 0..63: the 32 E2M1 codes (low nibble
//     first) of row (l % 16), block (l / 16) of the chunk, i.e. K range
//     [32 (l / 16), +32);
//   byte 1024 + l: that block's E8M0 scale.
// A wave loads an atom with one 16-byte and one 1-byte load per lane.  Word
// j of a lane's 16 bytes feeds MFMA step j of v_mfma_f32_16x16x32_bf16 as the
// B operand (hardware k = 8 (l / 16) + i stands for K = 32 (l / 16) + 8 j + i;
// the A operand uses the same correspondence, so the sum over K is exact).
// Gate and up are fused: row groups alternate 16 gate rows, 16 up rows
// (group 2p = gate rows 16p..16p+15, 2p+1 = up rows of the same indices).
// Record = [gate/up atoms: group-major, K-chunk minor] [down atoms: same].
// Total = 3*H*I*17/32 bytes, the MXFP4 size.
// ---------------------------------------------------------------------------
constexpr int kMaxH = 6144;            // largest hidden / inter size
constexpr int kMaxCacheSlots = 4096;   // the lookup keeps the LRU order in LDS
constexpr int kAtomRows = 16;
constexpr int kAtomK = 128;
constexpr int kAtomData = 1024;
constexpr int kAtomBytes = 1088;

// bf16 atom: the same 16 rows x 128 K tile as an MXFP4 atom, lane l's 32
// values (row l % 16, K block l / 16) as 4 pieces of 8 at 1024 p + 16 l.
constexpr int kAtomBytesBF16 = 4096;
inline size_t expert_record_bytes(int H, int I, int fmt = MOE_WEIGHTS_MXFP4) {
  return fmt == MOE_WEIGHTS_BF16 ? (size_t)3 * H * I * 2 : (size_t)3 * H * I * 17 / 32;
}
inline size_t gateup_section_bytes(int H, int I, int fmt = MOE_WEIGHTS_MXFP4) {
  return fmt == MOE_WEIGHTS_BF16 ? (size_t)2 * I * H * 2 : (size_t)2 * I * H * 17 / 32;
}

// Host-side repack of one canonical MXFP4 matrix [N][K] into atoms.
// fuse_pair: the matrix is gate (even groups) / up (odd groups) pair; pass
// both sources.  Out must hold N*K*17/32 (or twice that for fused) bytes.
void repack_gateup(const uint8_t* qg, const uint8_t* sg, const uint8_t* qu,
                   const uint8_t* su, int I, int H, uint8_t* out);
void repack_down(const uint8_t* qd, const uint8_t* sd, int H, int I, uint8_t* out);

// ---------------------------------------------------------------------------
// Device-side work descriptors written by the routing kernels.
// ---------------------------------------------------------------------------
struct WorkItem {          // one expert's share of a decode call
  const uint8_t* w;        // expert record (cache slot, staging or shared)
  int32_t pos0;            // first row in the permuted order
  int32_t cnt;             // rows (tokens) routed to it
};

struct FillEntry {         // one host-pool -> HBM expert copy
  const uint8_t* src;      // pinned host record (device-mapped)
  uint8_t* dst;            // cache or staging slot
};

// Small per-call counters kept on the device.
struct DevMeta {
  int32_t T;
  int32_t n_unique;
  int32_t n_items;
  int32_t n_fill;
  int32_t n_hit;
  int32_t n_bypass;
  int32_t pad[2];
};

// Cache state and statistics on the device.
struct DevCache {
  uint64_t clock;
  uint64_t lookups, hits, fills, bypasses, evictions;
};

// Arguments of the block-wide LRU lookup.
// Recency-order entry: slot | (key + 1) << kOrderKeyShift (key + 1 = 0: empty).
constexpr int kOrderKeyShift = 12;   // slots < 4096

struct LookupArgs {
  int32_t layer, E, C, staging;
  int32_t slot0;           // first slot this lookup may fill (C slots from it)
  int32_t insert;          // 0: misses bypass (the static policy's lookups)
  int32_t* key;            // [C]
  uint64_t* stamp;         // [C]
  int32_t* order;          // [C] packed entries, least recent first (the
                           // sub-array of the slots slot0 .. slot0+C-1)
  int32_t* order_tmp;      // [C]
  int32_t* map;            // [L*E] slot of each key or -1
  uint8_t* hitflag;        // [C]
  int32_t* victim;         // [max unique]
  DevCache* cache;
  const uint8_t* pool;     // pinned host pool (device-mapped)
  uint8_t* slots;          // [C] records
  uint8_t* staging_buf;    // [S] records
  size_t stride;           // bytes between records
  FillEntry* fills;        // [max unique]
  DevMeta* meta;
};

// ---------------------------------------------------------------------------
// Context
// ---------------------------------------------------------------------------
struct Ctx {
  moe_config cfg{};
  int device = 0;
  size_t rec_bytes = 0;     // 3*H*I*17/32
  size_t stride = 0;        // record stride (256-byte multiple)
  int max_unique = 0;       // min(T_max*k, E)
  int max_items = 0;        // max_unique + has_shared
  int rows_max = 0;         // T_max*k + T_max (shared rows)

  // host pool and HBM weights
  uint8_t* pool = nullptr;          // pinned, [L][E] records
  float* d_router = nullptr;        // [L][E][H]: router matrices, transposed
  uint8_t* d_shared = nullptr;      // [L] records
  std::vector<uint8_t> router_set;  // per layer
  std::vector<uint8_t> shared_set;

  // cache
  int C = 0;
  uint8_t* d_slots = nullptr;       // [C] records
  uint8_t* d_staging = nullptr;     // [S] records
  int32_t* d_key = nullptr;
  uint64_t* d_stamp = nullptr;
  int32_t* d_order = nullptr;
  int32_t* d_order_tmp = nullptr;
  uint8_t* d_hitflag = nullptr;
  int32_t* d_map = nullptr;         // [L*E]
  int32_t* d_victim = nullptr;
  DevCache* d_cache = nullptr;

  // decode scratch
  float* d_logits = nullptr;        // [T_max][E]
  int32_t* d_ids = nullptr;         // [T_max*k]
  float* d_gates = nullptr;         // [T_max*k]
  int32_t* d_counts = nullptr;      // [E]
  int32_t* d_offsets = nullptr;     // [E+1]
  int32_t* d_sorted = nullptr;      // [T_max*k]
  int32_t* d_inv = nullptr;         // [T_max*k]
  int32_t* d_unique = nullptr;      // [E]
  int32_t* d_slotcode = nullptr;    // [E]
  int32_t* d_tok = nullptr;         // [rows_max] token of each permuted row
  WorkItem* d_items = nullptr;      // [max_items]
  FillEntry* d_fills = nullptr;     // [max_unique]
  DevMeta* d_meta = nullptr;
  uint16_t* d_h = nullptr;          // bf16 [2][rows_max][I]: hi, lo planes
  float* d_yperm = nullptr;         // [rows_max][H]
  int32_t* d_lookup_ids = nullptr;  // [E] for expert_cache_fill

  // prefill (allocated on first use)
  int Tp_max = 0;
  uint8_t* d_layerbuf[2] = {nullptr, nullptr};
  hipStream_t copy_stream = nullptr;
  hipEvent_t ev_upload[2] = {nullptr, nullptr};
  hipEvent_t ev_compute[2] = {nullptr, nullptr};
  struct Prefill* pf = nullptr;

  // timing
  bool timing = false;
  std::vector<hipEvent_t> ev_pool;  // reused
  // start and stop of the gate/up and the down kernel, recorded by the
  // dispatches themselves
  struct TimingRec {
    hipEvent_t gu0, gu1, dn0, dn1;
  };
  std::vector<TimingRec> t_decode, t_prefill;
  size_t ev_next = 0;

  // host-side counters not tracked on the device
  moe_stats host_stats{};
};

// ---------------------------------------------------------------------------
// Launchers (each enqueues on `st` and returns hipGetLastError()).
// ---------------------------------------------------------------------------
hipError_t launch_router(const uint16_t* x, int T, int H, int E, const float* w_router_t,
                         const float* bias, float* logits, hipStream_t st);
hipError_t launch_route_finalize(Ctx* c, int layer, int T, int32_t* user_ids,
                                 float* user_gates, hipStream_t st);
hipError_t launch_cache_lookup(Ctx* c, int layer, const int32_t* d_experts,
                               const int32_t* d_n, int n_max, int32_t* d_slot, bool insert,
                               hipStream_t st);
hipError_t launch_fill(const FillEntry* fills, const DevMeta* meta, int max_fill,
                       size_t bytes, hipStream_t st);
hipError_t launch_copy_pairs(const FillEntry* pairs, int n, size_t bytes,
                             hipStream_t st);
hipError_t launch_probe_copy(const void* src, void* dst, size_t n_bytes,
                             hipStream_t st);
// The expert launchers take optional start and stop events: when given, the
// kernel is launched with hipExtLaunchKernel, which records them as part of
// the dispatch, so that their interval is the kernel's own duration.
hipError_t launch_expert_gateup(const Ctx* c, const uint16_t* x, int T, hipStream_t st,
                                hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_expert_down(const Ctx* c, int T, hipStream_t st, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr);
hipError_t launch_combine(const Ctx* c, int T, uint16_t* y, float* y32, hipStream_t st);
hipError_t launch_combine_rows(const float* yperm, const int32_t* inv, const float* gates, int T,
                               int k, int H, int has_shared, uint16_t* y, float* y32,
                               hipStream_t st);

// Next event of the context's timing pool (created on demand; NULL on failure).
hipEvent_t timing_event(Ctx* c);

// kernel<<<grid, block, shm, st>>>(args...), or with start and stop events
// recorded by the dispatch itself when ev0 is given.
#define MOE_LAUNCH(KERNEL, GRID, BLOCK, SHM, ST, EV0, EV1, ...)                          \
  do {                                                                                  \
    if (EV0)                                                                            \
      hipExtLaunchKernelGGL(KERNEL, dim3(GRID), dim3(BLOCK), (uint32_t)(SHM), ST, EV0, EV1, \
                            0u, __VA_ARGS__);                                           \
    else                                                                                \
      KERNEL<<<GRID, BLOCK, SHM, ST>>>(__VA_ARGS__);                                    \
  } while (0)

// Slots a lookup of `layer` may fill under the context's cache policy: the
// first one in *slot0 (may be NULL), the count returned.  insert = false for
// lookups that place nothing under the static policy (forward, lookup).
int fillable_slots(const Ctx* c, int layer, bool insert, int* slot0);

// prefill
int prefill_max_tiles(int T, int k, int E);
size_t prefill_lo_bytes(int T, int k, int E, int I);
hipError_t prefill_inspect(Ctx* c, int32_t* T, int32_t* ids, float* gates);
hipError_t prefill_forward(Ctx* c, int n_layers, const void* const* x, int T,
                           const float* const* bias, void* const* y, float* const* y32,
                           hipStream_t st);
void prefill_free(Ctx* c);

}  // namespace moe
