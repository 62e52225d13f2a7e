// Internal declarations of libmoe: context, device layouts, kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "layout.h"

namespace moe {

constexpr int kMaxH = 6144;            // largest hidden / inter size
constexpr int kMaxCacheSlots = 4096;   // the lookup keeps the LRU order in LDS

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
// Expert record size from which decode runs its copies on the copy stream
// beside the resident experts' kernels.
constexpr size_t kSplitFillMinBytes = size_t(4) << 20;

struct DevMeta {
  int32_t T;
  int32_t n_unique;
  int32_t n_items;         // work-list entries: unique experts + shared
  int32_t n_fill;          // copies issued (cache fills + bypasses)
  int32_t n_hit;
  int32_t n_bypass;
  int32_t zero;            // 0: the first item of the whole list and of the hit part
  int32_t n_items_a;       // items[0, n_items_a): resident experts and the shared
                           // one; items[n_items_a, n_items): experts copied by
                           // this call (fills and bypasses)
};

// Per-call device arrays of the decode forward, carved out of one buffer
// (decode_scratch_layout): the context's own, sized at create for
// max_tokens, or a caller-independent static one.
struct DecodeScratch {
  int T_cap = 0;             // tokens the layout was sized for
  int max_unique = 0;        // min(T_cap * k, E)
  int max_items = 0;         // max_unique + has_shared
  int rows_cap = 0;          // T_cap * k + T_cap (shared rows)
  size_t lo_plane = 0;       // elements from h's hi plane to its lo plane
  float* logits = nullptr;   // [T_cap][E]
  int32_t* ids = nullptr;    // [T_cap*k]
  float* gates = nullptr;    // [T_cap*k]
  int32_t* counts = nullptr;   // [E]
  int32_t* offsets = nullptr;  // [E+1]
  int32_t* sorted = nullptr;   // [T_cap*k]
  int32_t* inv = nullptr;      // [T_cap*k]
  int32_t* unique = nullptr;   // [E]
  int32_t* slotcode = nullptr; // [E]
  int32_t* tok = nullptr;      // [rows_cap] token of each permuted row
  WorkItem* items = nullptr;   // [max_items]
  FillEntry* fills = nullptr;  // [max_unique]
  DevMeta* meta = nullptr;
  uint16_t* h = nullptr;       // bf16 [2][rows_cap][I]: hi, lo planes
  float* yperm = nullptr;      // [rows_cap][H]
};

// Bytes of a decode scratch for T tokens; with base != NULL the arrays of
// *s are laid out from base (256-byte aligned pieces).
size_t decode_scratch_layout(const moe_config& f, int T, uint8_t* base, DecodeScratch* s);

// The fixed device scratch of moe_layer_forward_noalloc: its size, and the
// device address of `device`'s copy (resolved once per device, with that
// device current; later calls return the kept address).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch_address(int device, uint8_t** out);

// Cache state and statistics on the device.
struct DevCache {
  uint64_t clock;
  uint64_t lookups, hits, fills, bypasses, evictions;
  uint64_t pf_lookups, pf_hits, pf_fills;  // prefetch lookups (moe_set_prefetch)
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
  int32_t* map;            // [L*E] slot of each key or -1
  DevCache* cache;
  const uint8_t* pool;     // pinned host pool (device-mapped)
  uint8_t* slots;          // [C] records
  uint8_t* staging_buf;    // [S] records
  size_t stride;           // bytes between records
  FillEntry* fills;        // [max unique]
  DevMeta* meta;
  // A prefetch (moe_set_prefetch) when non-null: the meta of the call that
  // issues it, whose hit and filled slots (the most recent entries of the
  // recency order) are never victims; misses with no victim are skipped.
  const DevMeta* pin = nullptr;
};

// ---------------------------------------------------------------------------
// Cache slot memory: a device address range reserved for the largest
// capacity, backed by equal chunks (64 MiB .. 1 GiB, chosen per context)
// mapped from its start as far as the current capacity needs (HIP virtual
// memory management).
// ---------------------------------------------------------------------------
constexpr size_t kSlotChunkMin = (size_t)64 << 20;
constexpr size_t kSlotChunkMax = (size_t)1 << 30;
struct SlotArena {
  uint8_t* base = nullptr;
  size_t reserved = 0;     // bytes of address range
  size_t chunk = 0;        // bytes per physical chunk
  int device = 0;
  std::vector<hipMemGenericAllocationHandle_t> chunks;  // chunk i backs [i, i+1) * chunk
};
hipError_t arena_init(SlotArena& a, int device, size_t max_bytes);
// Back [0, bytes) with memory; all or nothing (on failure the arena is as before).
hipError_t arena_ensure(SlotArena& a, size_t bytes);
// Release the chunks that lie wholly at or past `bytes`.
void arena_trim(SlotArena& a, size_t bytes);
void arena_free(SlotArena& a);

// ---------------------------------------------------------------------------
// Context
// ---------------------------------------------------------------------------
struct Ctx {
  moe_config cfg{};
  int device = 0;
  size_t rec_bytes = 0;     // 3*H*I*17/32
  size_t stride = 0;        // record stride (256-byte multiple)

  // host pool and HBM weights
  uint8_t* pool = nullptr;          // pinned, [L][E] records
  float* d_router = nullptr;        // [L][E][H]: router matrices, transposed
  uint8_t* d_shared = nullptr;      // [L] records
  std::vector<uint8_t> router_set;  // per layer
  std::vector<uint8_t> shared_set;

  // cache: C slots of the arena; the state arrays hold max_slots entries so
  // that a resize never reallocates them
  int C = 0;
  int max_slots = 0;                // min(L*E, kMaxCacheSlots)
  SlotArena arena;
  uint8_t* d_slots = nullptr;       // arena.base: slot s at d_slots + s*stride
  uint8_t* d_staging = nullptr;     // [S] records
  int32_t* d_key = nullptr;         // [max_slots]
  uint64_t* d_stamp = nullptr;      // [max_slots]
  int32_t* d_order = nullptr;       // [max_slots]
  int32_t* d_map = nullptr;         // [L*E]
  FillEntry* d_pairs = nullptr;     // [max_slots] resize moves
  DevCache* d_cache = nullptr;

  // decode scratch (one allocation, sized for max_tokens), and the device
  // address of this device's fixed scratch array (moe_layer_forward_noalloc)
  uint8_t* d_scratch = nullptr;
  DecodeScratch ds;
  uint8_t* static_scratch = nullptr;
  int32_t* d_lookup_ids = nullptr;  // [E] for expert_cache_fill

  // internal stream of the prefill layer uploads and of the decode kernels
  // of resident experts that run beside a call's fills, joined to the
  // caller's stream by events
  hipStream_t copy_stream = nullptr;
  bool split_fills = false;         // decode computes resident experts beside the fills
                                    // (expert records of kSplitFillMinBytes and more)
  hipEvent_t ev_routed = nullptr;   // decode: the work and fill lists are written
  hipEvent_t ev_resident = nullptr; // decode: the resident experts are computed

  // cross-layer prefetch: the request armed by moe_set_prefetch (consumed
  // by the next decode call), the stream its lookup and copies run on beside
  // that call's expert kernels and into the next call, its fill list and
  // meta, and the events that order it against later cache work
  struct PrefetchReq {
    int layer = -1;
    const int32_t* experts = nullptr;
    int n = 0;
  } pf_req;
  hipStream_t pf_stream = nullptr;
  FillEntry* d_pf_fills = nullptr;  // [E]
  DevMeta* d_pf_meta = nullptr;
  hipEvent_t ev_filled = nullptr;   // the issuing call's own copies are done
  hipEvent_t ev_pf_lookup = nullptr;  // the prefetch's cache-state update is done
  hipEvent_t ev_pf_done = nullptr;  // its copies are done
  bool pf_inflight = false;         // a prefetch ran on pf_stream that no later
                                    // cache work has waited for yet
  uint64_t* pf_flag = nullptr;      // pinned host word: the last prefetch whose
  uint64_t pf_seq = 0;              // copies are done (the device stores pf_seq)

  // prefill (allocated on first use)
  int prefill_format = MOE_PREFILL_BF16;
  int Tp_max = 0;
  uint8_t* d_layerbuf[2] = {nullptr, nullptr};
  hipEvent_t ev_upload[2] = {nullptr, nullptr};
  hipEvent_t ev_compute[2] = {nullptr, nullptr};
  struct Prefill* pf = nullptr;

  // timing: start and stop events of each stage, recorded by the kernel
  // dispatches themselves
  bool timing = false;
  std::vector<hipEvent_t> ev_pool;  // reused
  struct TimingRec {
    hipEvent_t ev[2 * 8];
    bool split = false;  // decode call that ran its expert kernels in two parts
  };
  std::vector<TimingRec> t_decode, t_prefill;
  size_t ev_next = 0;

  // host-side counters not tracked on the device
  moe_stats host_stats{};

  // debug switches (MOE_DEBUG_*), and the state after a failed copy: slots
  // may name experts whose bytes did not land, so cache work is refused
  // until expert_cache_reset
  int debug_flags = 0;
  bool failed = false;
};

// ---------------------------------------------------------------------------
// Launchers (each enqueues on `st` and returns hipGetLastError()).  Every
// launcher takes optional start and stop events (either may be NULL): when
// one is given, the kernel is launched with hipExtLaunchKernel, which
// records them as part of the dispatch, so that their interval is the
// kernel's own duration.
// ---------------------------------------------------------------------------
hipError_t launch_router(const uint16_t* x, int T, int H, int E, const float* w_router_t,
                         const float* bias, float* logits, hipStream_t st,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_route_finalize(Ctx* c, const DecodeScratch& s, int layer, int T,
                                 int32_t* user_ids, float* user_gates, hipStream_t st,
                                 hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_cache_lookup(Ctx* c, int layer, const int32_t* d_experts,
                               const int32_t* d_n, int n_max, int32_t* d_slot, bool insert,
                               hipStream_t st);
// prefetch lookup of d_experts[0..n) of `layer` into d_pf_fills / d_pf_meta,
// pinning what the call whose meta is `pin` uses
hipError_t launch_cache_prefetch(Ctx* c, int layer, const int32_t* d_experts, int n,
                                 const DevMeta* pin, hipStream_t st);
// confined: the fill runs beside expert kernels (few workgroups, each
// holding its CU's LDS so that no expert-kernel workgroup shares the CU)
hipError_t launch_fill(const FillEntry* fills, const DevMeta* meta, int max_fill,
                       size_t bytes, bool confined, hipStream_t st, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr);
hipError_t launch_copy_pairs(const FillEntry* pairs, int n, size_t bytes,
                             hipStream_t st);
// store seq to *host_flag (pinned host memory) once the stream gets there
hipError_t launch_signal(uint64_t* host_flag, uint64_t seq, hipStream_t st);
hipError_t launch_probe_copy(const void* src, void* dst, size_t n_bytes,
                             hipStream_t st);
// What one launch of the expert kernels covers: items [*lo_p, *hi_p) of a
// work list, the token of each permuted row, h (two bf16 planes, lo_plane
// elements apart) and the fp32 expert outputs.
struct ExpertList {
  const WorkItem* items = nullptr;
  int items_cap = 0;                // entries of items[]
  const int32_t* lo_p = nullptr;    // device bounds of the items covered
  const int32_t* hi_p = nullptr;
  int grid_items = 0;               // grid rows: the most items the bounds can hold
  int split_items = 0;              // items the K split is chosen for (the whole list)
  const int32_t* tok = nullptr;     // permuted row -> token
  uint16_t* h = nullptr;
  size_t lo_plane = 0;
  float* yperm = nullptr;
  bool stream = false;              // at most 16 rows per item: the streaming kernels
};
hipError_t launch_gateup_list(const Ctx* c, const ExpertList& L, const uint16_t* x,
                              uint32_t x_bytes, hipStream_t st, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr);
hipError_t launch_down_list(const Ctx* c, const ExpertList& L, hipStream_t st,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Which part of the work list an expert-kernel launch covers: all items,
// the resident experts and the shared one, or the experts this call copies.
enum ItemRange { kItemsAll, kItemsResident, kItemsCopied };
hipError_t launch_expert_gateup(const Ctx* c, const DecodeScratch& s, const uint16_t* x, int T,
                                ItemRange part, hipStream_t st, hipEvent_t ev0 = nullptr,
                                hipEvent_t ev1 = nullptr);
hipError_t launch_expert_down(const Ctx* c, const DecodeScratch& s, int T, ItemRange part,
                              hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_combine_rows(const float* yperm, const int32_t* inv, const float* gates, int T,
                               int k, int H, int has_shared, uint16_t* y, float* y32,
                               hipStream_t st, hipEvent_t ev0 = nullptr,
                               hipEvent_t ev1 = nullptr);

// Next event of the context's timing pool (created on demand; NULL on failure).
hipEvent_t timing_event(Ctx* c);

// Stages timed per decode call and per prefill layer.  A decode call whose
// fills run beside the resident experts' kernels times the second part of
// gate/up and down as stages of their own (kStGateUpB, kStDownB), summed into
// gate/up and down when reported.
enum DecodeStage { kStRouter, kStFinalize, kStFill, kStGateUp, kStDown, kStCombine, kDecodeStages,
                   kStGateUpB = kDecodeStages, kStDownB, kDecodeTimed };
enum PrefillStage { kPfRouting, kPfGateUp, kPfDown, kPfCombine, kPrefillStages };

// kernel<<<grid, block, shm, st>>>(args...), or with start and stop events
// recorded by the dispatch itself when either is given.
#define MOE_LAUNCH(KERNEL, GRID, BLOCK, SHM, ST, EV0, EV1, ...)                          \
  do {                                                                                  \
    if ((EV0) || (EV1))                                                                 \
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
int prefill_layers_run(const Ctx* c);
// 1 if the last prefill call ran in the MXFP8 mode, 0 if not, -1 if none ran
int prefill_last_mx(const Ctx* c);
hipError_t prefill_inspect_mx(Ctx* c, int32_t* T, uint8_t* xq, uint8_t* xs, uint8_t* hq,
                              uint8_t* hs);
hipError_t prefill_inspect(Ctx* c, int layer, int32_t* T, int32_t* ids, float* gates,
                           int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* inv);
hipError_t prefill_forward(Ctx* c, int n_layers, const void* const* x, int T,
                           const float* const* bias, void* const* y, float* const* y32,
                           hipStream_t st);
void prefill_free(Ctx* c);

}  // namespace moe
