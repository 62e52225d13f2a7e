// C-ABI entry points of libmoe: validation, memory ownership, cache state,
// and the launch sequence of the decode forward.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

#include "moe_internal.h"
#include "repack.h"
#include "resize_plan.h"

using namespace moe;

namespace {

// The last error message of this thread, in a fixed buffer (reporting an
// error allocates nothing).
thread_local char g_err[512];

moe_status fail(moe_status code, const char* msg) {
  std::snprintf(g_err, sizeof g_err, "%s", msg);
  return code;
}
moe_status fail(moe_status code, const std::string& msg) { return fail(code, msg.c_str()); }

#define HIPCHK(expr)                                                        \
  do {                                                                      \
    hipError_t _e = (expr);                                                 \
    if (_e != hipSuccess) {                                                 \
      std::snprintf(g_err, sizeof g_err, "%s: %s", #expr,                   \
                    hipGetErrorString(_e));                                 \
      return MOE_ERR_HIP;                                                   \
    }                                                                       \
  } while (0)

#define ALLOC(ptr, bytes)                                                   \
  do {                                                                      \
    size_t _b = (bytes);                                                    \
    if (_b) {                                                               \
      hipError_t _e = hipMalloc((void**)&(ptr), _b);                        \
      if (_e != hipSuccess) {                                               \
        destroy_all(c);                                                     \
        return fail(MOE_ERR_OOM, std::string("hipMalloc ") + #ptr + " (" +  \
                                     std::to_string(_b) + " bytes): " +     \
                                     hipGetErrorString(_e));                \
      }                                                                     \
    }                                                                       \
  } while (0)

template <class T>
void dfree(T*& p) {
  if (p) (void)hipFree((void*)p);
  p = nullptr;
}

void destroy_all(Ctx* c) {
  if (!c) return;
  prefill_free(c);
  if (c->pool) (void)hipHostFree(c->pool);
  c->pool = nullptr;
  dfree(c->d_router); dfree(c->d_shared); dfree(c->d_staging);
  arena_free(c->arena);
  c->d_slots = nullptr;
  dfree(c->d_key); dfree(c->d_stamp); dfree(c->d_order); dfree(c->d_map); dfree(c->d_pairs);
  dfree(c->d_cache);
  dfree(c->d_scratch);
  c->ds = DecodeScratch{};
  dfree(c->d_lookup_ids);
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  c->ev_pool.clear();
  if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
  c->copy_stream = nullptr;
  if (c->ev_routed) (void)hipEventDestroy(c->ev_routed);
  if (c->ev_resident) (void)hipEventDestroy(c->ev_resident);
  c->ev_routed = c->ev_resident = nullptr;
  if (c->pf_stream) (void)hipStreamDestroy(c->pf_stream);
  c->pf_stream = nullptr;
  if (c->ev_filled) (void)hipEventDestroy(c->ev_filled);
  if (c->ev_pf_lookup) (void)hipEventDestroy(c->ev_pf_lookup);
  if (c->ev_pf_done) (void)hipEventDestroy(c->ev_pf_done);
  c->ev_filled = c->ev_pf_lookup = c->ev_pf_done = nullptr;
  dfree(c->d_pf_fills);
  dfree(c->d_pf_meta);
  if (c->pf_flag) (void)hipHostFree(c->pf_flag);
  c->pf_flag = nullptr;
}

bool scales_valid(const uint8_t* s, size_t n) {
  for (size_t i = 0; i < n; i++)
    if (s[i] == 255) return false;
  return true;
}

// Upload a host vector to a device array (sync).
template <class T>
hipError_t upload(T* dst, const std::vector<T>& v) {
  if (v.empty()) return hipSuccess;
  return hipMemcpy(dst, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
}

moe_status check_ctx(moe_ctx* ctx) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  return MOE_OK;
}

Ctx* C_(moe_ctx* ctx) { return reinterpret_cast<Ctx*>(ctx); }


constexpr size_t kMaxTimingPairs = 65536;

}  // namespace

namespace moe {

size_t decode_scratch_layout(const moe_config& f, int T, uint8_t* base, DecodeScratch* s) {
  const int H = f.hidden, I = f.inter, E = f.n_experts, k = f.top_k;
  DecodeScratch d;
  d.T_cap = T;
  d.max_unique = std::min(T * k, E);
  d.max_items = d.max_unique + f.has_shared;
  d.rows_cap = T * k + T;
  d.lo_plane = (size_t)d.rows_cap * I;
  size_t off = 0;
  auto take = [&](auto*& ptr, size_t bytes) {
    using P = std::remove_reference_t<decltype(ptr)>;
    ptr = base ? reinterpret_cast<P>(base + off) : nullptr;
    off += (bytes + 255) / 256 * 256;
  };
  take(d.logits, (size_t)T * E * 4);
  take(d.ids, (size_t)T * k * 4);
  take(d.gates, (size_t)T * k * 4);
  take(d.counts, (size_t)E * 4);
  take(d.offsets, (size_t)(E + 1) * 4);
  take(d.sorted, (size_t)T * k * 4);
  take(d.inv, (size_t)T * k * 4);
  take(d.unique, (size_t)E * 4);
  take(d.slotcode, (size_t)E * 4);
  take(d.tok, (size_t)d.rows_cap * 4);
  take(d.items, (size_t)d.max_items * sizeof(WorkItem));
  take(d.fills, (size_t)d.max_unique * sizeof(FillEntry));
  take(d.meta, sizeof(DevMeta));
  take(d.h, (size_t)d.rows_cap * I * 2 * 2);  // hi and lo bf16 planes
  take(d.yperm, (size_t)d.rows_cap * H * 4);
  if (s) *s = d;
  return off;
}

int fillable_slots(const Ctx* c, int layer, bool insert, int* slot0) {
  int first = 0, n = c->C;
  if (c->cfg.cache_policy == MOE_CACHE_PER_LAYER) {
    const int64_t L = c->cfg.n_layers;
    first = (int)(layer * (int64_t)c->C / L);
    n = (int)((layer + 1) * (int64_t)c->C / L) - first;
  } else if (c->cfg.cache_policy == MOE_CACHE_STATIC && !insert) {
    n = 0;
  }
  if (slot0) *slot0 = first;
  return n;
}

hipEvent_t timing_event(Ctx* c) {
  if (c->ev_next == c->ev_pool.size()) {
    hipEvent_t e;
    // Timing only: no system-scope fences (they flush caches and add
    // microseconds between the event and the kernel it brackets).
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    c->ev_pool.push_back(e);
  }
  return c->ev_pool[c->ev_next++];
}

// Repack one expert into `rec` in the context's format.
static void repack_expert(const Ctx* c, const uint8_t* qg, const uint8_t* qu, const uint8_t* qd,
                          const uint8_t* sg, const uint8_t* su, const uint8_t* sd, uint8_t* rec) {
  repack_record(c->cfg.weight_format, c->cfg.hidden, c->cfg.inter, qg, qu, qd, sg, su, sd, rec);
}

}  // namespace moe

namespace {

// The decode forward of one layer on the scratch s (T <= s.T_cap), all on
// the caller's stream: router -> finalize (top-k, dispatch, cache lookup,
// work list, fill list) -> copies of this call's misses from the pinned
// pool (cache fills and bypasses) -> gate/up + SwiGLU -> down -> combine.
// The copies of a decode call or a cache fill.  A copy that fails (or the
// injected failure of MOE_DEBUG_FAIL_NEXT_FILL) leaves slots that name
// experts whose bytes did not land: the context then refuses cache work
// until expert_cache_reset.
static moe_status issue_fill(Ctx* c, const FillEntry* fills, const DevMeta* meta, int max_fill,
                             bool confined, hipStream_t st, hipEvent_t ev0 = nullptr,
                             hipEvent_t ev1 = nullptr) {
  if (c->debug_flags & MOE_DEBUG_FAIL_NEXT_FILL) {
    c->debug_flags &= ~MOE_DEBUG_FAIL_NEXT_FILL;
    c->failed = true;
    return fail(MOE_ERR_HIP,
                "fill: injected failure, the copies were not issued (expert_cache_reset "
                "empties the cache)");
  }
  const hipError_t e = launch_fill(fills, meta, max_fill, c->rec_bytes, confined, st, ev0, ev1);
  if (e != hipSuccess) {
    c->failed = true;
    return fail(MOE_ERR_HIP, std::string("fill: ") + hipGetErrorString(e) +
                                 " (expert_cache_reset empties the cache)");
  }
  return MOE_OK;
}

// Wait for all work on the device; a prefetch in flight is then done.
static hipError_t sync_device(Ctx* c) {
  const hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) c->pf_inflight = false;
  return e;
}

// Make `st` wait for a prefetch still in flight (its cache-state update and
// its copies) before cache work queued on it next.
static hipError_t join_prefetch(Ctx* c, hipStream_t st) {
  if (!c->pf_inflight) return hipSuccess;
  const hipError_t e = hipStreamWaitEvent(st, c->ev_pf_done, 0);
  if (e == hipSuccess) c->pf_inflight = false;
  return e;
}

// MOE_DEBUG_SYNC: wait for the streams a stage used and check for errors,
// naming the stage.
static moe_status debug_sync(Ctx* c, hipStream_t st, bool both, bool capturing, const char* stage) {
  if (!(c->debug_flags & MOE_DEBUG_SYNC) || capturing) return MOE_OK;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess && both) e = hipStreamSynchronize(c->copy_stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, std::string(stage) + ": " + hipGetErrorString(e));
  return MOE_OK;
}

moe_status decode_forward(Ctx* c, const DecodeScratch& s, int layer, const uint16_t* x, int T,
                          const float* bias, uint16_t* y, float* y32, int32_t* ids,
                          float* gates, hipStream_t st, bool allow_timing) {
  const moe_config& f = c->cfg;
  const Ctx::PrefetchReq pr = c->pf_req;  // consumed by this call
  c->pf_req = Ctx::PrefetchReq{};
  // The resident experts' kernels run beside the copies of the missed ones
  // when one expert's copy is long (split_fills); not under stream capture,
  // where the whole call stays on one stream.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIPCHK(hipStreamIsCapturing(st, &cs));
  const bool capturing = cs != hipStreamCaptureStatusNone;
  const bool split = c->split_fills && !capturing;
  Ctx::TimingRec tr{};
  tr.split = split;
  const bool timed = allow_timing && c->timing && c->t_decode.size() < kMaxTimingPairs;
  if (timed)
    for (int i = 0; i < 2 * (split ? kDecodeTimed : kDecodeStages); i++)
      if (!(tr.ev[i] = timing_event(c))) return fail(MOE_ERR_HIP, "timing event");
  auto t0 = [&](int stage) { return timed ? tr.ev[2 * stage] : nullptr; };
  auto t1 = [&](int stage) { return timed ? tr.ev[2 * stage + 1] : nullptr; };
  auto done = [&](bool both, const char* stage) { return debug_sync(c, st, both, capturing, stage); };
  const float* wr = c->d_router + (size_t)layer * f.hidden * f.n_experts;
  const int max_fill = std::min(T * f.top_k, f.n_experts);
  // A prefetch issued by the previous call may still be copying: its cache
  // update must precede this call's lookup, and its copies this call's
  // copies and expert kernels (the router runs meanwhile).  Under capture
  // it must be over already (waiting on it cannot be recorded).
  if (c->pf_inflight && __atomic_load_n(c->pf_flag, __ATOMIC_ACQUIRE) >= c->pf_seq)
    c->pf_inflight = false;  // its copies are done
  const bool pf_wait = c->pf_inflight;
  if (pf_wait && capturing)
    return fail(MOE_ERR_STATE,
                "a prefetch issued by an earlier call is still copying; synchronize the device "
                "before capturing");
  HIPCHK(launch_router(x, T, f.hidden, f.n_experts, wr, bias, s.logits, st, t0(kStRouter),
                       t1(kStRouter)));
  if (moe_status r = done(false, "router")) return r;
  if (pf_wait && !capturing) HIPCHK(hipStreamWaitEvent(st, c->ev_pf_lookup, 0));
  HIPCHK(launch_route_finalize(c, s, layer, T, ids, gates, st, t0(kStFinalize),
                               t1(kStFinalize)));
  if (moe_status r = done(false, "finalize")) return r;
  if (pf_wait && !capturing) HIPCHK(join_prefetch(c, st));
  // A prefetch armed by moe_set_prefetch: looked up and copied once this
  // call's own copies are done, beside its expert kernels and into the next
  // call (on the prefetch stream; the next cache work waits for it), or
  // under capture in order on `stream`.
  auto prefetch = [&]() -> moe_status {
    if (pr.n <= 0) return MOE_OK;
    hipStream_t ps = capturing ? st : c->pf_stream;
    if (!capturing) {
      HIPCHK(hipEventRecord(c->ev_filled, st));
      HIPCHK(hipStreamWaitEvent(ps, c->ev_filled, 0));
    }
    HIPCHK(launch_cache_prefetch(c, pr.layer, pr.experts, pr.n, s.meta, ps));
    if (!capturing) HIPCHK(hipEventRecord(c->ev_pf_lookup, ps));
    if (moe_status r = issue_fill(c, c->d_pf_fills, c->d_pf_meta, pr.n, true, ps)) return r;
    if (!capturing) {
      HIPCHK(hipEventRecord(c->ev_pf_done, ps));
      HIPCHK(launch_signal(c->pf_flag, ++c->pf_seq, ps));
      c->pf_inflight = true;
    }
    return debug_sync(c, ps, false, capturing, "prefetch");
  };
  if (split) {
    // The fills follow finalize on `stream`, so that their workgroups are
    // placed first; the resident experts run on the internal stream once
    // the lists exist (its event wait delays them behind the fill's
    // dispatch); the copied experts run on `stream` after both.
    HIPCHK(hipEventRecord(c->ev_routed, st));
    if (moe_status r = issue_fill(c, s.fills, s.meta, max_fill, true, st, t0(kStFill), t1(kStFill))) return r;
    if (moe_status r = done(false, "fill")) return r;
    if (moe_status r = prefetch()) return r;
    HIPCHK(hipStreamWaitEvent(c->copy_stream, c->ev_routed, 0));
    HIPCHK(launch_expert_gateup(c, s, x, T, kItemsResident, c->copy_stream, t0(kStGateUp),
                                t1(kStGateUp)));
    if (moe_status r = done(true, "gate/up (resident experts)")) return r;
    HIPCHK(launch_expert_down(c, s, T, kItemsResident, c->copy_stream, t0(kStDown), t1(kStDown)));
    if (moe_status r = done(true, "down (resident experts)")) return r;
    HIPCHK(hipEventRecord(c->ev_resident, c->copy_stream));
    HIPCHK(hipStreamWaitEvent(st, c->ev_resident, 0));
    HIPCHK(launch_expert_gateup(c, s, x, T, kItemsCopied, st, t0(kStGateUpB), t1(kStGateUpB)));
    if (moe_status r = done(false, "gate/up (copied experts)")) return r;
    HIPCHK(launch_expert_down(c, s, T, kItemsCopied, st, t0(kStDownB), t1(kStDownB)));
    if (moe_status r = done(false, "down (copied experts)")) return r;
  } else {
    if (moe_status r = issue_fill(c, s.fills, s.meta, max_fill, false, st, t0(kStFill), t1(kStFill))) return r;
    if (moe_status r = done(false, "fill")) return r;
    if (moe_status r = prefetch()) return r;
    HIPCHK(launch_expert_gateup(c, s, x, T, kItemsAll, st, t0(kStGateUp), t1(kStGateUp)));
    if (moe_status r = done(false, "gate/up")) return r;
    HIPCHK(launch_expert_down(c, s, T, kItemsAll, st, t0(kStDown), t1(kStDown)));
    if (moe_status r = done(false, "down")) return r;
  }
  HIPCHK(launch_combine_rows(s.yperm, s.inv, s.gates, T, f.top_k, f.hidden, f.has_shared, y, y32,
                             st, t0(kStCombine), t1(kStCombine)));
  if (moe_status r = done(false, "combine")) return r;
  if (timed) c->t_decode.push_back(tr);
  return MOE_OK;
}

}  // namespace

// =========================================================================
extern "C" {

const char* moe_last_error(void) { return g_err; }

size_t moe_expert_bytes(int32_t hidden, int32_t inter) {
  if (hidden <= 0 || inter <= 0) return 0;
  return expert_record_bytes(hidden, inter);
}

moe_status moe_create(const moe_config* cfg, moe_ctx** out) {
  if (!cfg || !out) return fail(MOE_ERR_INVALID_ARG, "cfg and out must not be NULL");
  const moe_config& f = *cfg;
  if (f.hidden <= 0 || f.inter <= 0 || f.n_layers < 1 || f.top_k < 1 || f.top_k > 16 ||
      f.n_experts < f.top_k || f.n_experts > 1024 || f.max_tokens < 1 ||
      f.max_tokens > 64 || f.cache_slots < 0 || f.staging_slots < 0 ||
      f.max_prefill_tokens < 0 || (f.has_shared != 0 && f.has_shared != 1) ||
      f.cache_policy < MOE_CACHE_GLOBAL || f.cache_policy > MOE_CACHE_STATIC ||
      f.weight_format < MOE_WEIGHTS_MXFP4 || f.weight_format > MOE_WEIGHTS_NVFP4 ||
      f.prefill_format < MOE_PREFILL_BF16 || f.prefill_format > MOE_PREFILL_MXFP8 ||
      (f.renormalize != 0 && f.renormalize != 1))
    return fail(MOE_ERR_INVALID_ARG, "moe_config field out of range");
  if ((int64_t)f.cache_slots > (int64_t)f.n_layers * f.n_experts)
    return fail(MOE_ERR_INVALID_ARG, "cache_slots exceeds n_layers*n_experts");
  if ((int64_t)f.n_layers * f.n_experts >= (1 << (31 - kOrderKeyShift)))
    return fail(MOE_ERR_UNSUPPORTED, "n_layers*n_experts too large");
  if (f.hidden % 128 || f.inter % 128 || f.hidden > kMaxH || f.inter > kMaxH)
    return fail(MOE_ERR_UNSUPPORTED, "hidden and inter must be multiples of 128, at most 6144");
  if (f.weight_format == MOE_WEIGHTS_BF16 && f.max_tokens > 16 &&
      (f.hidden > 4096 || f.inter > 4096))
    return fail(MOE_ERR_UNSUPPORTED,
                "bf16 experts above 16 tokens per decode call need H and I <= 4096");
  if (f.prefill_format == MOE_PREFILL_MXFP8 && f.weight_format != MOE_WEIGHTS_MXFP4)
    return fail(MOE_ERR_UNSUPPORTED, "the MXFP8 prefill mode needs MXFP4 experts");
  if (f.cache_slots > kMaxCacheSlots)
    return fail(MOE_ERR_UNSUPPORTED, "cache_slots above 4096");
  if (f.max_prefill_tokens > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "max_prefill_tokens too large");
  // The prefill kernels address x (T x H bf16), h (a bf16 plane of
  // T*(k+1) x I) and h's low-order records through 32-bit buffer offsets.
  if ((int64_t)f.max_prefill_tokens * f.hidden * 2 >= (int64_t(1) << 31) ||
      (int64_t)f.max_prefill_tokens * (f.top_k + 1) * f.inter * 2 >= (int64_t(1) << 31) ||
      (int64_t)prefill_lo_bytes(f.max_prefill_tokens, f.top_k, f.n_experts, f.inter) >=
          (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED,
                "max_prefill_tokens too large for this shape (x or h reach 2 GiB)");

  Ctx* c = new (std::nothrow) Ctx();
  if (!c) return fail(MOE_ERR_OOM, "context allocation");
  c->cfg = f;
  {
    const hipError_t e0 = hipGetDevice(&c->device);
    if (e0 != hipSuccess) {
      delete c;
      return fail(MOE_ERR_HIP, std::string("device query: ") + hipGetErrorString(e0));
    }
  }
  const int H = f.hidden, I = f.inter, E = f.n_experts, L = f.n_layers;
  const int Tm = f.max_tokens;
  c->rec_bytes = expert_record_bytes(H, I, f.weight_format);
  c->stride = (c->rec_bytes + 255) / 256 * 256;
  c->C = f.cache_slots;
  c->prefill_format = f.prefill_format;
  c->router_set.assign(L, 0);
  c->shared_set.assign(L, 0);

  const size_t pool_bytes = (size_t)L * E * c->stride;
  hipError_t e = hipHostMalloc((void**)&c->pool, pool_bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    c->pool = nullptr;
    destroy_all(c);
    delete c;
    return fail(MOE_ERR_OOM, "pinned host pool of " + std::to_string(pool_bytes) +
                                 " bytes: " + hipGetErrorString(e));
  }
  ALLOC(c->d_router, (size_t)L * H * E * sizeof(float));
  if (f.has_shared) ALLOC(c->d_shared, (size_t)L * c->stride);
  c->max_slots = (int)std::min<int64_t>((int64_t)L * E, kMaxCacheSlots);
  {
    hipError_t ea = arena_init(c->arena, c->device, (size_t)c->max_slots * c->stride);
    if (ea == hipSuccess) ea = arena_ensure(c->arena, (size_t)c->C * c->stride);
    if (ea != hipSuccess) {
      destroy_all(c);
      delete c;
      return fail(ea == hipErrorOutOfMemory ? MOE_ERR_OOM : MOE_ERR_HIP,
                  std::string("cache slot memory: ") + hipGetErrorString(ea));
    }
    c->d_slots = c->arena.base;
  }
  ALLOC(c->d_staging, (size_t)f.staging_slots * c->stride);
  ALLOC(c->d_key, (size_t)c->max_slots * 4);
  ALLOC(c->d_stamp, (size_t)c->max_slots * 8);
  ALLOC(c->d_order, (size_t)c->max_slots * 4);
  ALLOC(c->d_map, (size_t)L * E * 4);
  ALLOC(c->d_pairs, (size_t)c->max_slots * sizeof(FillEntry));
  ALLOC(c->d_cache, sizeof(DevCache));
  ALLOC(c->d_scratch, decode_scratch_layout(f, Tm, nullptr, nullptr));
  decode_scratch_layout(f, Tm, c->d_scratch, &c->ds);
  ALLOC(c->d_lookup_ids, (size_t)(E + 1) * 4);
  ALLOC(c->d_pf_fills, (size_t)E * sizeof(FillEntry));
  ALLOC(c->d_pf_meta, sizeof(DevMeta));
  if (hipHostMalloc((void**)&c->pf_flag, 64, hipHostMallocDefault) != hipSuccess) {
    c->pf_flag = nullptr;
    destroy_all(c);
    delete c;
    return fail(MOE_ERR_OOM, "pinned prefetch flag");
  }
  *c->pf_flag = 0;
  {
    // default priority (the caller's streams are expected to use it too)
    hipError_t es = hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking);
    if (es == hipSuccess) es = hipStreamCreateWithFlags(&c->pf_stream, hipStreamNonBlocking);
    // the decode events order work between streams of this device only:
    // no timing, no system-scope release
    const unsigned ef = hipEventDisableTiming | hipEventDisableSystemFence;
    if (es == hipSuccess) es = hipEventCreateWithFlags(&c->ev_routed, ef);
    if (es == hipSuccess) es = hipEventCreateWithFlags(&c->ev_resident, ef);
    if (es == hipSuccess) es = hipEventCreateWithFlags(&c->ev_filled, ef);
    if (es == hipSuccess) es = hipEventCreateWithFlags(&c->ev_pf_lookup, ef);
    if (es == hipSuccess) es = hipEventCreateWithFlags(&c->ev_pf_done, ef);
    if (es != hipSuccess) {
      destroy_all(c);
      delete c;
      return fail(MOE_ERR_HIP, std::string("copy stream: ") + hipGetErrorString(es));
    }
    // decode copies beside the resident experts' kernels once one expert's
    // copy (hundreds of microseconds at 4 MiB and more over PCIe) dwarfs the
    // cost of the extra launches and event waits
    c->split_fills = c->rec_bytes >= kSplitFillMinBytes;
  }

  std::vector<int32_t> key(std::max(c->C, 1), -1), order(std::max(c->C, 1)), map((size_t)L * E, -1);
  std::iota(order.begin(), order.end(), 0);  // all empty: slot | (0 << kOrderKeyShift)
  std::vector<uint64_t> stamp(std::max(c->C, 1), 0);
  std::vector<uint8_t> zero(sizeof(DevCache) > sizeof(DevMeta) ? sizeof(DevCache) : sizeof(DevMeta), 0);
  if (upload(c->d_key, key) != hipSuccess || upload(c->d_order, order) != hipSuccess ||
      upload(c->d_stamp, stamp) != hipSuccess || upload(c->d_map, map) != hipSuccess ||
      hipMemcpy(c->d_cache, zero.data(), sizeof(DevCache), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->ds.meta, zero.data(), sizeof(DevMeta), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->d_pf_meta, zero.data(), sizeof(DevMeta), hipMemcpyHostToDevice) != hipSuccess) {
    destroy_all(c);
    delete c;
    return fail(MOE_ERR_HIP, "initialising cache state");
  }
  {
    const hipError_t es = static_scratch_address(c->device, &c->static_scratch);
    if (es != hipSuccess) {
      destroy_all(c);
      delete c;
      return fail(MOE_ERR_HIP, std::string("device scratch address: ") + hipGetErrorString(es));
    }
  }
  *out = reinterpret_cast<moe_ctx*>(c);
  g_err[0] = 0;
  return MOE_OK;
}

moe_status moe_destroy(moe_ctx* ctx) {
  if (!ctx) return MOE_OK;
  Ctx* c = C_(ctx);
  (void)hipDeviceSynchronize();
  destroy_all(c);
  delete c;
  return MOE_OK;
}

moe_status moe_set_router(moe_ctx* ctx, int32_t layer, const float* h_router) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (layer < 0 || layer >= c->cfg.n_layers || !h_router)
    return fail(MOE_ERR_INVALID_ARG, "bad layer or NULL router");
  const size_t H = c->cfg.hidden, E = c->cfg.n_experts;
  std::vector<float> t(H * E);  // [E][H]: one expert's column contiguous
  for (size_t h = 0; h < H; h++)
    for (size_t e = 0; e < E; e++) t[e * H + h] = h_router[h * E + e];
  HIPCHK(hipMemcpy(c->d_router + (size_t)layer * H * E, t.data(), H * E * 4,
                   hipMemcpyHostToDevice));
  c->router_set[layer] = 1;
  return MOE_OK;
}

moe_status moe_set_expert(moe_ctx* ctx, int32_t layer, int32_t expert,
                          const uint8_t* qg, const uint8_t* qu, const uint8_t* qd,
                          const uint8_t* sg, const uint8_t* su, const uint8_t* sd) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const int H = c->cfg.hidden, I = c->cfg.inter;
  if (layer < 0 || layer >= c->cfg.n_layers || expert < -1 || expert >= c->cfg.n_experts)
    return fail(MOE_ERR_INVALID_ARG, "bad layer or expert index");
  const bool bf16 = c->cfg.weight_format == MOE_WEIGHTS_BF16;
  const bool nv = c->cfg.weight_format == MOE_WEIGHTS_NVFP4;
  if (!qg || !qu || !qd || (!bf16 && (!sg || !su || !sd)))
    return fail(MOE_ERR_INVALID_ARG, "NULL weight pointer");
  if (bf16 && (sg || su || sd))
    return fail(MOE_ERR_INVALID_ARG, "bf16 experts take no scale arrays");
  if (expert == -1 && !c->cfg.has_shared)
    return fail(MOE_ERR_STATE, "context has no shared expert");
  if (nv) {
    const size_t n16 = (size_t)H * I / 16;
    for (const uint8_t* s : {sg, su, sd}) {
      for (size_t i = 0; i < n16; i++)
        if ((s[i] & 0x80) || s[i] == 0x7F)
          return fail(MOE_ERR_INVALID_ARG, "E4M3 block scale negative or NaN");
      float t;
      std::memcpy(&t, s + n16, 4);
      if (!std::isfinite(t)) return fail(MOE_ERR_INVALID_ARG, "matrix scale not finite");
    }
  } else if (!bf16) {
    const size_t ns = (size_t)H * I / 32;
    if (!scales_valid(sg, ns) || !scales_valid(su, ns) || !scales_valid(sd, ns))
      return fail(MOE_ERR_INVALID_ARG, "E8M0 scale byte 255 (NaN)");
  }
  if (expert >= 0) {
    uint8_t* rec = c->pool + ((size_t)layer * c->cfg.n_experts + expert) * c->stride;
    repack_expert(c, qg, qu, qd, sg, su, sd, rec);
    return MOE_OK;
  }
  std::vector<uint8_t> rec(c->stride, 0);
  repack_expert(c, qg, qu, qd, sg, su, sd, rec.data());
  HIPCHK(hipMemcpy(c->d_shared + (size_t)layer * c->stride, rec.data(), c->stride,
                   hipMemcpyHostToDevice));
  c->shared_set[layer] = 1;
  return MOE_OK;
}

moe_status moe_set_layer(moe_ctx* ctx, int32_t layer, const float* h_router,
                         const uint8_t* h_q, const uint8_t* h_s,
                         const uint8_t* h_shared_q, const uint8_t* h_shared_s) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const bool bf16 = c->cfg.weight_format == MOE_WEIGHTS_BF16;
  if (layer < 0 || layer >= c->cfg.n_layers || !h_router || !h_q || (!bf16 && !h_s))
    return fail(MOE_ERR_INVALID_ARG, "bad layer or NULL pointer");
  if (bf16 && (h_s || h_shared_s)) return fail(MOE_ERR_INVALID_ARG, "bf16 experts take no scales");
  if (c->cfg.has_shared && (!h_shared_q || (!bf16 && !h_shared_s)))
    return fail(MOE_ERR_INVALID_ARG, "shared expert weights required");
  const size_t H = c->cfg.hidden, I = c->cfg.inter;
  const bool nv = c->cfg.weight_format == MOE_WEIGHTS_NVFP4;
  const size_t q1 = bf16 ? H * I * 2 : H * I / 2;
  const size_t s1 = bf16 ? 0 : nv ? H * I / 16 + 4 : H * I / 32;
  auto sp = [&](const uint8_t* base, size_t off) { return base ? base + off : nullptr; };
  if (moe_status s = moe_set_router(ctx, layer, h_router)) return s;
  for (int e = 0; e < c->cfg.n_experts; e++) {
    const uint8_t* q = h_q + (size_t)e * 3 * q1;
    const uint8_t* s = sp(h_s, (size_t)e * 3 * s1);
    if (moe_status st = moe_set_expert(ctx, layer, e, q, q + q1, q + 2 * q1, s, sp(s, s1),
                                       sp(s, 2 * s1)))
      return st;
  }
  if (c->cfg.has_shared)
    return moe_set_expert(ctx, layer, -1, h_shared_q, h_shared_q + q1, h_shared_q + 2 * q1,
                          h_shared_s, sp(h_shared_s, s1), sp(h_shared_s, 2 * s1));
  return MOE_OK;
}

// Checks shared by the two decode entry points (messages without
// allocation).  Returns MOE_OK or the failure to report.
static const char kFailedMsg[] =
    "a copy of an expert failed earlier; expert_cache_reset empties the cache";

static moe_status check_forward(Ctx* c, int32_t layer, const void* d_x, int32_t T,
                                const void* d_y) {
  const moe_config& f = c->cfg;
  if (c->failed) return fail(MOE_ERR_STATE, kFailedMsg);
  if (layer < 0 || layer >= f.n_layers) return fail(MOE_ERR_INVALID_ARG, "bad layer");
  if (T < 0 || T > f.max_tokens) return fail(MOE_ERR_INVALID_ARG, "T outside [0, max_tokens]");
  if (T == 0) return MOE_OK;
  if (!d_x || !d_y) return fail(MOE_ERR_INVALID_ARG, "NULL x or y");
  if (!c->router_set[layer]) return fail(MOE_ERR_STATE, "router of this layer not set");
  if (f.has_shared && !c->shared_set[layer])
    return fail(MOE_ERR_STATE, "shared expert of this layer not set");
  const int worst_bypass =
      std::max(0, std::min(T * f.top_k, f.n_experts) - fillable_slots(c, layer, false, nullptr));
  if (worst_bypass > f.staging_slots) {
    std::snprintf(g_err, sizeof g_err, "staging_slots (%d) below worst-case bypass count %d",
                  f.staging_slots, worst_bypass);
    return MOE_ERR_CAPACITY;
  }
  return MOE_OK;
}

moe_status moe_layer_forward(moe_ctx* ctx, int32_t layer, const void* d_x, int32_t T,
                             const float* d_bias, void* d_y, float* d_y32, int32_t* d_ids,
                             float* d_gates, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (moe_status s = check_forward(c, layer, d_x, T, d_y)) return s;
  if (T == 0) return MOE_OK;
  if (moe_status s = decode_forward(c, c->ds, layer, (const uint16_t*)d_x, T, d_bias,
                                    (uint16_t*)d_y, d_y32, d_ids, d_gates, (hipStream_t)stream,
                                    true))
    return s;
  c->host_stats.forward_calls++;
  return MOE_OK;
}

moe_status moe_layer_forward_noalloc(moe_ctx* ctx, int32_t layer, const void* d_x, int32_t T,
                                     const float* d_bias, void* d_y, float* d_y32,
                                     int32_t* d_ids, float* d_gates, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (moe_status s = check_forward(c, layer, d_x, T, d_y)) return s;
  if (T == 0) return MOE_OK;
  const size_t need = decode_scratch_layout(c->cfg, T, nullptr, nullptr);
  if (need > kStaticScratchBytes) {
    std::snprintf(g_err, sizeof g_err,
                  "this call needs %zu bytes of device scratch, the fixed array holds %zu",
                  need, kStaticScratchBytes);
    return MOE_ERR_CAPACITY;
  }
  DecodeScratch s;
  decode_scratch_layout(c->cfg, T, c->static_scratch, &s);
  if (moe_status st = decode_forward(c, s, layer, (const uint16_t*)d_x, T, d_bias,
                                     (uint16_t*)d_y, d_y32, d_ids, d_gates, (hipStream_t)stream,
                                     false))
    return st;
  c->host_stats.forward_calls++;
  return MOE_OK;
}

moe_status moe_prefill_forward(moe_ctx* ctx, int32_t n_layers, const void* const* h_x,
                               int32_t T, const float* const* h_bias, void* const* h_y,
                               float* const* h_y32, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const moe_config& f = c->cfg;
  if (f.max_prefill_tokens == 0) return fail(MOE_ERR_STATE, "prefill disabled (max_prefill_tokens = 0)");
  if (n_layers < 1 || n_layers > f.n_layers || !h_x || !h_y)
    return fail(MOE_ERR_INVALID_ARG, "bad n_layers or NULL pointer arrays");
  if (T < 1 || T > f.max_prefill_tokens) return fail(MOE_ERR_INVALID_ARG, "T outside [1, max_prefill_tokens]");
  for (int l = 0; l < n_layers; l++) {
    if (!h_x[l] || !h_y[l]) return fail(MOE_ERR_INVALID_ARG, "NULL x or y pointer");
    if (!c->router_set[l]) return fail(MOE_ERR_STATE, "router not set");
    if (f.has_shared && !c->shared_set[l]) return fail(MOE_ERR_STATE, "shared expert not set");
  }
  hipError_t e = prefill_forward(c, n_layers, h_x, T, h_bias, h_y, h_y32, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(MOE_ERR_UNSUPPORTED, "prefill path not available");
  if (e == hipErrorOutOfMemory) return fail(MOE_ERR_OOM, "prefill buffers");
  HIPCHK(e);
  c->host_stats.prefill_layers += n_layers;
  return MOE_OK;
}

moe_status moe_set_prefill_format(moe_ctx* ctx, int32_t format) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (format < MOE_PREFILL_BF16 || format > MOE_PREFILL_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "unknown prefill format");
  if (format == MOE_PREFILL_MXFP8 && c->cfg.weight_format != MOE_WEIGHTS_MXFP4)
    return fail(MOE_ERR_UNSUPPORTED, "the MXFP8 prefill mode needs MXFP4 experts");
  HIPCHK(sync_device(c));
  c->prefill_format = format;
  return MOE_OK;
}

moe_status expert_cache_lookup(moe_ctx* ctx, int32_t layer, const int32_t* d_experts,
                               const int32_t* d_n, int32_t* d_slot, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (c->failed) return fail(MOE_ERR_STATE, kFailedMsg);
  if (layer < 0 || layer >= c->cfg.n_layers || !d_experts || !d_n || !d_slot)
    return fail(MOE_ERR_INVALID_ARG, "bad layer or NULL pointer");
  const int worst_bypass = std::max(0, c->ds.max_unique - fillable_slots(c, layer, false, nullptr));
  if (worst_bypass > c->cfg.staging_slots)
    return fail(MOE_ERR_CAPACITY, "staging_slots below worst-case bypass count");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(join_prefetch(c, st));
  HIPCHK(launch_cache_lookup(c, layer, d_experts, d_n, c->ds.max_unique, d_slot, false, st));
  return issue_fill(c, c->ds.fills, c->ds.meta, c->ds.max_unique, false, st);
}

moe_status expert_cache_fill(moe_ctx* ctx, int32_t layer, const int32_t* h_experts,
                             int32_t n, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (c->failed) return fail(MOE_ERR_STATE, kFailedMsg);
  if (layer < 0 || layer >= c->cfg.n_layers || n < 0 || n > c->ds.max_unique ||
      (n > 0 && !h_experts))
    return fail(MOE_ERR_INVALID_ARG, "bad layer, count or NULL list");
  for (int i = 0; i < n; i++) {
    if (h_experts[i] < 0 || h_experts[i] >= c->cfg.n_experts)
      return fail(MOE_ERR_INVALID_ARG, "expert id out of range");
    if (i && h_experts[i] <= h_experts[i - 1])
      return fail(MOE_ERR_INVALID_ARG, "expert ids must be ascending and unique");
  }
  if (n == 0) return MOE_OK;
  if (std::max(0, n - fillable_slots(c, layer, true, nullptr)) > c->cfg.staging_slots)
    return fail(MOE_ERR_CAPACITY, "fill would bypass more experts than staging_slots");
  hipStream_t st = (hipStream_t)stream;
  std::vector<int32_t> buf(h_experts, h_experts + n);
  buf.push_back(n);
  HIPCHK(join_prefetch(c, st));
  HIPCHK(hipStreamSynchronize(st));
  HIPCHK(hipMemcpy(c->d_lookup_ids, buf.data(), buf.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(launch_cache_lookup(c, layer, c->d_lookup_ids, c->d_lookup_ids + n, n, c->ds.slotcode,
                             true, st));
  if (moe_status r = issue_fill(c, c->ds.fills, c->ds.meta, n, false, st)) return r;
  HIPCHK(hipStreamSynchronize(st));
  return MOE_OK;
}

// Upload a slot table (and the expert -> slot map it implies) for C2 slots.
static hipError_t upload_cache_state(Ctx* c, const std::vector<int32_t>& key,
                                     const std::vector<uint64_t>& stamp,
                                     const std::vector<int32_t>& order) {
  const int L = c->cfg.n_layers, E = c->cfg.n_experts;
  std::vector<int32_t> map((size_t)L * E, -1);
  for (size_t s = 0; s < key.size(); s++)
    if (key[s] >= 0) map[key[s]] = (int32_t)s;
  hipError_t e = upload(c->d_key, key);
  if (e == hipSuccess) e = upload(c->d_stamp, stamp);
  if (e == hipSuccess) e = upload(c->d_order, order);
  if (e == hipSuccess) e = upload(c->d_map, map);
  return e;
}

moe_status expert_cache_resize(moe_ctx* ctx, int32_t new_slots, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const int L = c->cfg.n_layers, E = c->cfg.n_experts;
  if (c->failed) return fail(MOE_ERR_STATE, kFailedMsg);
  if (new_slots < 0 || (int64_t)new_slots > (int64_t)L * E)
    return fail(MOE_ERR_INVALID_ARG, "new_slots outside [0, n_layers*n_experts]");
  if (new_slots > kMaxCacheSlots) return fail(MOE_ERR_UNSUPPORTED, "cache_slots above 4096");
  if (c->cfg.cache_policy != MOE_CACHE_GLOBAL)
    return fail(MOE_ERR_UNSUPPORTED, "resize is supported for the global cache policy only");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(hipStreamSynchronize(st));
  HIPCHK(sync_device(c));
  const int C = c->C, C2 = new_slots;
  std::vector<int32_t> key(C);
  std::vector<uint64_t> stamp(C);
  DevCache dc;
  if (C) {
    HIPCHK(hipMemcpy(key.data(), c->d_key, (size_t)C * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(stamp.data(), c->d_stamp, (size_t)C * 8, hipMemcpyDeviceToHost));
  }
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));
  const ResizePlan plan = plan_resize(key, stamp, C2, kOrderKeyShift);

  // Growing maps memory for the new slots first: on failure nothing changed.
  if (C2 > C) {
    const hipError_t e = arena_ensure(c->arena, (size_t)C2 * c->stride);
    if (e != hipSuccess)
      return fail(e == hipErrorOutOfMemory ? MOE_ERR_OOM : MOE_ERR_HIP,
                  std::string("cache slot memory: ") + hipGetErrorString(e));
  }
  // Shrinking moves the survivors held past the new capacity down (sources
  // and destinations are disjoint) and only then publishes the new table.
  // Should that fail part way, the records the old table names may already
  // be overwritten, so the cache is left empty (always consistent: outputs
  // never depend on the cache) and the error is returned.
  auto fail_empty = [&](hipError_t e) {
    const std::vector<int32_t> k0(C2, -1);
    const std::vector<uint64_t> s0(C2, 0);
    (void)upload_cache_state(c, k0, s0, recency_order(k0, s0, kOrderKeyShift));
    c->C = C2;
    std::snprintf(g_err, sizeof g_err, "resize: %s (the cache was emptied)", hipGetErrorString(e));
    return MOE_ERR_HIP;
  };
  if (!plan.moves.empty()) {
    std::vector<FillEntry> pairs;
    for (const auto& m : plan.moves)
      pairs.push_back({c->d_slots + (size_t)m.first * c->stride, c->d_slots + (size_t)m.second * c->stride});
    hipError_t e = hipMemcpy(c->d_pairs, pairs.data(), pairs.size() * sizeof(FillEntry),
                             hipMemcpyHostToDevice);
    if (e == hipSuccess) e = launch_copy_pairs(c->d_pairs, (int)pairs.size(), c->rec_bytes, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail_empty(e);
  }
  if (hipError_t e = upload_cache_state(c, plan.key, plan.stamp, plan.order)) return fail_empty(e);
  dc.evictions += plan.evicted.size();
  if (hipError_t e = hipMemcpy(c->d_cache, &dc, sizeof dc, hipMemcpyHostToDevice)) return fail_empty(e);
  c->C = C2;
  if (C2 < C) arena_trim(c->arena, (size_t)C2 * c->stride);
  c->host_stats.resizes++;
  c->host_stats.bytes_d2d += (uint64_t)plan.moves.size() * c->rec_bytes;
  return MOE_OK;
}

moe_status expert_cache_reset(moe_ctx* ctx) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  HIPCHK(sync_device(c));
  const int C = std::max(c->C, 1);
  std::vector<int32_t> key(C, -1), order(C);
  std::iota(order.begin(), order.end(), 0);  // all empty: slot | (0 << kOrderKeyShift)
  std::vector<uint64_t> stamp(C, 0);
  HIPCHK(upload_cache_state(c, key, stamp, order));
  HIPCHK(sync_device(c));
  c->failed = false;
  return MOE_OK;
}

moe_status moe_set_debug(moe_ctx* ctx, int32_t flags) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (flags & ~(MOE_DEBUG_SYNC | MOE_DEBUG_FAIL_NEXT_FILL))
    return fail(MOE_ERR_INVALID_ARG, "unknown debug flag");
  C_(ctx)->debug_flags = flags;
  return MOE_OK;
}

moe_status expert_cache_snapshot(moe_ctx* ctx, int32_t capacity, int32_t* h_key,
                                 uint64_t* h_stamp, uint64_t* h_clock, int32_t* h_slots) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (!h_slots) return fail(MOE_ERR_INVALID_ARG, "h_slots is NULL");
  *h_slots = c->C;
  if (capacity < c->C) return fail(MOE_ERR_CAPACITY, "snapshot capacity below cache size");
  if ((c->C && (!h_key || !h_stamp)) || !h_clock)
    return fail(MOE_ERR_INVALID_ARG, "NULL snapshot array");
  HIPCHK(sync_device(c));
  if (c->C) {
    HIPCHK(hipMemcpy(h_key, c->d_key, (size_t)c->C * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(h_stamp, c->d_stamp, (size_t)c->C * 8, hipMemcpyDeviceToHost));
  }
  DevCache dc;
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));
  *h_clock = dc.clock;
  return MOE_OK;
}

moe_status moe_inspect_dispatch(moe_ctx* ctx, int32_t* h_T, int32_t* h_counts,
                                int32_t* h_offsets, int32_t* h_sorted, int32_t* h_inv,
                                int32_t* h_unique, int32_t* h_n_unique, int32_t* h_slot) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  HIPCHK(sync_device(c));
  const DecodeScratch& d = c->ds;
  DevMeta m;
  HIPCHK(hipMemcpy(&m, d.meta, sizeof m, hipMemcpyDeviceToHost));
  const int E = c->cfg.n_experts, nk = m.T * c->cfg.top_k;
  if (h_T) *h_T = m.T;
  if (h_n_unique) *h_n_unique = m.n_unique;
  if (h_counts) HIPCHK(hipMemcpy(h_counts, d.counts, (size_t)E * 4, hipMemcpyDeviceToHost));
  if (h_offsets) HIPCHK(hipMemcpy(h_offsets, d.offsets, (size_t)(E + 1) * 4, hipMemcpyDeviceToHost));
  if (h_sorted && nk) HIPCHK(hipMemcpy(h_sorted, d.sorted, (size_t)nk * 4, hipMemcpyDeviceToHost));
  if (h_inv && nk) HIPCHK(hipMemcpy(h_inv, d.inv, (size_t)nk * 4, hipMemcpyDeviceToHost));
  if (h_unique && m.n_unique)
    HIPCHK(hipMemcpy(h_unique, d.unique, (size_t)m.n_unique * 4, hipMemcpyDeviceToHost));
  if (h_slot && m.n_unique)
    HIPCHK(hipMemcpy(h_slot, d.slotcode, (size_t)m.n_unique * 4, hipMemcpyDeviceToHost));
  return MOE_OK;
}

moe_status moe_inspect_prefill(moe_ctx* ctx, int32_t layer, int32_t* h_T, int32_t* h_ids,
                               float* h_gates, int32_t* h_counts, int32_t* h_offsets,
                               int32_t* h_sorted, int32_t* h_inv) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (!h_T) return fail(MOE_ERR_INVALID_ARG, "h_T is NULL");
  Ctx* c = C_(ctx);
  const int run = prefill_layers_run(c);
  if (run > 0 && (layer < 0 || layer >= run))
    return fail(MOE_ERR_INVALID_ARG, "layer outside the layers of the last prefill call");
  HIPCHK(prefill_inspect(c, layer, h_T, h_ids, h_gates, h_counts, h_offsets, h_sorted, h_inv));
  return MOE_OK;
}

moe_status moe_inspect_prefill_mx(moe_ctx* ctx, int32_t* h_T, uint8_t* h_xq, uint8_t* h_xs,
                                  uint8_t* h_hq, uint8_t* h_hs) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (!h_T) return fail(MOE_ERR_INVALID_ARG, "h_T is NULL");
  Ctx* c = C_(ctx);
  if (prefill_last_mx(c) == 0)
    return fail(MOE_ERR_UNSUPPORTED, "the last prefill call did not run in the MXFP8 mode");
  HIPCHK(prefill_inspect_mx(c, h_T, h_xq, h_xs, h_hq, h_hs));
  return MOE_OK;
}

moe_status moe_set_prefetch(moe_ctx* ctx, int32_t layer, const int32_t* d_experts,
                            int32_t n) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (c->failed) return fail(MOE_ERR_STATE, kFailedMsg);
  if (c->cfg.cache_policy != MOE_CACHE_GLOBAL)
    return fail(MOE_ERR_UNSUPPORTED, "prefetch is supported for the global cache policy only");
  if (layer < 0 || layer >= c->cfg.n_layers || n < 0 || n > c->cfg.n_experts ||
      (n > 0 && !d_experts))
    return fail(MOE_ERR_INVALID_ARG, "bad layer, count or NULL list");
  c->pf_req = n > 0 ? Ctx::PrefetchReq{layer, d_experts, n} : Ctx::PrefetchReq{};
  return MOE_OK;
}

moe_status moe_set_copy_overlap(moe_ctx* ctx, int32_t mode) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (mode < -1 || mode > 1) return fail(MOE_ERR_INVALID_ARG, "mode must be -1, 0 or 1");
  Ctx* c = C_(ctx);
  c->split_fills = mode == 1 || (mode == -1 && c->rec_bytes >= kSplitFillMinBytes);
  return MOE_OK;
}

moe_status moe_get_stats(moe_ctx* ctx, moe_stats* out) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  Ctx* c = C_(ctx);
  HIPCHK(sync_device(c));
  DevCache dc;
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));
  *out = c->host_stats;
  out->lookups = dc.lookups;
  out->hits = dc.hits;
  out->fills = dc.fills;
  out->bypasses = dc.bypasses;
  out->evictions = dc.evictions;
  out->prefetch_lookups = dc.pf_lookups;
  out->prefetch_hits = dc.pf_hits;
  out->prefetch_fills = dc.pf_fills;
  out->bytes_h2d = (dc.fills + dc.bypasses + dc.pf_fills) * c->rec_bytes;
  return MOE_OK;
}

moe_status moe_reset_stats(moe_ctx* ctx) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  HIPCHK(sync_device(c));
  DevCache dc;
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));
  const uint64_t clock = dc.clock;
  dc = DevCache{};
  dc.clock = clock;
  HIPCHK(hipMemcpy(c->d_cache, &dc, sizeof dc, hipMemcpyHostToDevice));
  c->host_stats = moe_stats{};
  return MOE_OK;
}

moe_status moe_set_timing(moe_ctx* ctx, int32_t enable) {
  if (moe_status s = check_ctx(ctx)) return s;
  C_(ctx)->timing = enable != 0;
  return MOE_OK;
}

// Stages that must have finished before a stage can start (-1 ends a
// list).  A stage's time is its stop minus the latest of its own start and
// its predecessors' stops, so that a dispatch-recorded start taken before
// the kernel could run does not count.
static const int kDecodePreds[kDecodeStages][3] = {
    {-1, -1, -1}, {kStRouter, -1, -1}, {kStFinalize, -1, -1},
    {kStFill, -1, -1}, {kStGateUp, -1, -1}, {kStDown, -1, -1}};
// a call whose fills run beside the resident experts' kernels
static const int kDecodeSplitPreds[kDecodeTimed][3] = {
    {-1, -1, -1}, {kStRouter, -1, -1}, {kStFinalize, -1, -1},
    {kStFinalize, -1, -1}, {kStGateUp, -1, -1}, {kStDownB, -1, -1},
    {kStDown, kStFill, -1}, {kStGateUpB, -1, -1}};
static const int kPrefillPreds[kPrefillStages][3] = {
    {-1, -1, -1}, {kPfRouting, -1, -1}, {kPfGateUp, -1, -1}, {kPfDown, -1, -1}};

// Time of stage i of record r: its stop minus the latest of its own start
// and its predecessors' stops.
static hipError_t stage_ms(const Ctx::TimingRec& r, int i, const int (*preds)[3], double* ms) {
  float t = 0;
  hipError_t e = hipEventElapsedTime(&t, r.ev[2 * i], r.ev[2 * i + 1]);
  for (int j = 0; j < 3 && e == hipSuccess && preds[i][j] >= 0; j++) {
    float u = 0;
    e = hipEventElapsedTime(&u, r.ev[2 * preds[i][j] + 1], r.ev[2 * i + 1]);
    t = std::min(t, u);
  }
  *ms = (double)std::max(t, 0.0f);
  return e;
}

// Sum the stage times of the records into ms[0..stages); the second parts
// of a split decode call's expert kernels count to gate/up and down.
static hipError_t sum_timing(const std::vector<Ctx::TimingRec>& v, int stages,
                             const int (*preds)[3], double* ms, bool decode) {
  for (int i = 0; i < stages; i++) ms[i] = 0.0;
  for (const auto& r : v) {
    const bool split = decode && r.split;
    const int (*pr)[3] = split ? kDecodeSplitPreds : preds;
    for (int i = 0; i < (split ? (int)kDecodeTimed : stages); i++) {
      double t = 0;
      if (hipError_t e = stage_ms(r, i, pr, &t)) return e;
      const int to = i == kStGateUpB ? kStGateUp : i == kStDownB ? kStDown : i;
      ms[split ? to : i] += t;
    }
  }
  return hipSuccess;
}

moe_status moe_get_timing(moe_ctx* ctx, moe_timing* out) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  Ctx* c = C_(ctx);
  HIPCHK(sync_device(c));
  double d[kDecodeStages], p[kPrefillStages];
  HIPCHK(sum_timing(c->t_decode, kDecodeStages, kDecodePreds, d, true));
  HIPCHK(sum_timing(c->t_prefill, kPrefillStages, kPrefillPreds, p, false));
  int n_split = 0;
  for (const auto& r : c->t_decode) n_split += r.split ? 1 : 0;
  *out = moe_timing{};
  out->n_decode = (int32_t)c->t_decode.size();
  out->n_prefill = (int32_t)c->t_prefill.size();
  out->n_decode_split = n_split;
  for (int i = 0; i < kDecodeStages; i++) out->decode_ms[i] = d[i];
  for (int i = 0; i < kPrefillStages; i++) out->prefill_ms[i] = p[i];
  c->t_decode.clear();
  c->t_prefill.clear();
  c->ev_next = 0;
  return MOE_OK;
}

moe_status moe_probe_copy(const void* d_src, void* d_dst, size_t n_bytes, void* stream) {
  if (!d_src || !d_dst || n_bytes % 16) return fail(MOE_ERR_INVALID_ARG, "bad copy arguments");
  if (!n_bytes) return MOE_OK;
  HIPCHK(launch_probe_copy(d_src, d_dst, n_bytes, (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"
