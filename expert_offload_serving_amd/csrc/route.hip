// Routing for the decode forward: router logits, top-k, gates, dispatch
// permutation and the global LRU cache lookup, all on the device.
//
// The router is unchanged by offloading (jansverre.net FreeToken article,
// section "Hva er FreeToken?"); the cache is one LRU shared by all MoE
// layers (same article, section "Hvorfor er båndbredden viktigere enn antall
// kjerner?"), exploiting overlap between adjacent tokens (aipolix.com
// FreeToken article, fifth paragraph).
#include "moe_internal.h"
#include "route_common.h"

namespace moe {
namespace {

constexpr int kRouterWaves = 4;       // waves per expert in the router
constexpr int kRouterTG = 8;          // tokens per pass
constexpr int kFinalizeThreads = 1024;

// logits[t][e] = fp32(sum_h x[t][h] W_r[h][e] + bias[t][e]), sums in fp64
// (bf16 x fp32 products are exact in fp64).  W_r is held transposed,
// [E][H], so an expert's column is contiguous.  One workgroup per expert:
// its 4 waves split H into quarters, lane l of a wave takes the 8-element
// pieces l, l+64, ... of its quarter (all loads issued before the first
// FMA), each wave reduces in a fixed DPP order and the quarters are added
// in order through LDS.
constexpr int kRouterMaxPieces = 3;   // pieces per lane: H <= 4 * 64 * 8 * 3

template <int TG>
__global__ __launch_bounds__(kRouterWaves * 64) void router_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E, const float* __restrict__ wrt,
    const float* __restrict__ bias, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x;
  const int per_wave = H / 8 / kRouterWaves;   // pieces in this wave's quarter
  const int q0 = w * per_wave;
  const float* wrow = wrt + (size_t)e * H;
  __shared__ double red[kRouterWaves][TG];
  f32x4 w0[kRouterMaxPieces], w1[kRouterMaxPieces];
#pragma unroll
  for (int i = 0; i < kRouterMaxPieces; i++) {
    const int q = lane + 64 * i;
    if (q < per_wave) {
      w0[i] = *reinterpret_cast<const f32x4*>(wrow + 8 * (q0 + q));
      w1[i] = *reinterpret_cast<const f32x4*>(wrow + 8 * (q0 + q) + 4);
    } else {
      w0[i] = w1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int tg = 0; tg < T; tg += TG) {
    const int tn = min(TG, T - tg);
    u32x4 xv[kRouterMaxPieces][TG];
#pragma unroll
    for (int i = 0; i < kRouterMaxPieces; i++) {
      const int q = lane + 64 * i;
#pragma unroll
      for (int t = 0; t < TG; t++)
        xv[i][t] = (q < per_wave && t < tn)
                       ? *reinterpret_cast<const u32x4*>(x + (size_t)(tg + t) * H + 8 * (q0 + q))
                       : u32x4{0u, 0u, 0u, 0u};
    }
    double acc[TG];
#pragma unroll
    for (int t = 0; t < TG; t++) acc[t] = 0.0;
#pragma unroll
    for (int i = 0; i < kRouterMaxPieces; i++) {
      double wd[8];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        wd[j] = (double)w0[i][j];
        wd[4 + j] = (double)w1[i][j];
      }
#pragma unroll
      for (int t = 0; t < TG; t++) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const uint32_t word = xv[i][t][j >> 1];
          const float xf = __uint_as_float((j & 1) ? (word & 0xFFFF0000u) : (word << 16));
          acc[t] = fma((double)xf, wd[j], acc[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TG; t++) {
      const double s = wave_sum_f64(acc[t]);
      if (lane == 0) red[w][t] = s;
    }
    lds_sync();
    if ((int)threadIdx.x < tn) {
      const int t = threadIdx.x;
      double s = 0.0;
#pragma unroll
      for (int v = 0; v < kRouterWaves; v++) s += red[v][t];
      const size_t o = (size_t)(tg + t) * E + e;
      logits[o] = (float)(bias ? s + (double)bias[o] : s);
    }
    lds_sync();
  }
}

// LDS working set of a lookup: the packed recency order, per-slot hit
// flags, the victims, and this layer's expert -> slot map.
struct LookupShared {
  int order[kMaxCacheSlots];
  uint8_t hit[kMaxCacheSlots];
  int victim[1024];
  int map[1024];
  int tmp[16];
  int evict;
  uint64_t clock0;
};

// Copy the recency order and this layer's map into LDS (issued first, so
// the loads overlap the work before the lookup).
__device__ __forceinline__ void prefetch_lookup(const LookupArgs& a, LookupShared& ls) {
  if (threadIdx.x == 0) ls.clock0 = a.cache->clock;
  for (int p = threadIdx.x; p < a.C; p += blockDim.x) ls.order[p] = a.order[p];
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) ls.map[e] = a.map[a.layer * a.E + e];
}

// Block-wide LRU lookup of the n unique experts in s_U (ascending).  Slot
// codes go to s_slot[u]; fills (cache and staging copies) to a.fills.  The
// rule is the one stated in moe.h (moe_layer_forward).  prefetch_lookup
// must have run (and a barrier passed) before.
__device__ void block_lookup(const LookupArgs& a, LookupShared& ls, const int* s_U, int n,
                             int* s_slot) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int C = a.C;
  const uint64_t clock0 = ls.clock0;
  if (tid == 0) ls.evict = 0;
  for (int s = tid; s < C; s += nt) ls.hit[a.slot0 + s] = 0;

  const int u = tid;
  const int e = u < n ? s_U[u] : -1;
  const bool valid = e >= 0 && e < a.E;
  const int key = valid ? a.layer * a.E + e : -1;
  const int slot = valid ? ls.map[e] : -1;
  const bool hit = valid && slot >= 0;
  const bool miss = valid && !hit;
  // One scan ranks hits (low 16 bits) and misses (high 16 bits): n <= 1024.
  int both;
  const int ranks = block_excl_scan((hit ? 1 : 0) | (miss ? 1 << 16 : 0), ls.tmp, &both);  // barrier: hit[] cleared
  const int hrank = ranks & 0xFFFF, mrank = ranks >> 16;
  const int n_hit = both & 0xFFFF, n_miss = both >> 16;
  // A prefetch leaves the issuing call's slots alone: they are the last
  // n_pin entries of the recency order (that call stamped them last, and
  // none holds a key of this lookup, which names another layer's experts or
  // experts that call did not use).
  const bool pf = a.pin != nullptr;
  const int n_pin = pf ? a.pin->n_hit + a.pin->n_fill - a.pin->n_bypass : 0;
  const int n_fill = a.insert ? max(0, min(n_miss, C - n_hit - n_pin)) : 0;
  if (hit) {
    ls.hit[slot] = 1;
    a.stamp[slot] = clock0 + 1 + (uint64_t)hrank;
    s_slot[u] = slot;
  }
  lds_sync();

  // Victims: the first n_fill non-hit slots in recency order; the other
  // non-hit slots are kept, compacted to the front in place (non-hit number
  // r goes to position r - n_fill, never above its own position, and every
  // position of a chunk is read before the chunk's first write).
  constexpr int kSlotMask = (1 << kOrderKeyShift) - 1;
  int carry = 0;
  for (int p0 = 0; p0 < C; p0 += nt) {
    const int p = p0 + tid;
    const int ent = p < C ? ls.order[p] : 0;
    const bool nonhit = p < C && !ls.hit[ent & kSlotMask];
    int tot;
    const int r = block_excl_scan(nonhit ? 1 : 0, ls.tmp, &tot) + carry;
    if (nonhit) {
      if (r < n_fill)
        ls.victim[r] = ent;
      else
        ls.order[r - n_fill] = ent;
    }
    carry += tot;
  }
  lds_sync();
  const int n_keep = C - n_hit - n_fill;
  if (hit) ls.order[n_keep + hrank] = slot | ((key + 1) << kOrderKeyShift);
  if (miss) {
    const uint8_t* src = a.pool + (size_t)key * a.stride;
    if (mrank < n_fill) {
      const int ent = ls.victim[mrank];
      const int s = ent & kSlotMask, old = (ent >> kOrderKeyShift) - 1;
      if (old >= 0) {
        a.map[old] = -1;
        atomicAdd(&ls.evict, 1);
      }
      a.key[s] = key;
      a.map[key] = s;
      a.stamp[s] = clock0 + (uint64_t)n_hit + 1 + (uint64_t)mrank;
      ls.order[n_keep + n_hit + mrank] = s | ((key + 1) << kOrderKeyShift);
      a.fills[mrank] = FillEntry{src, a.slots + (size_t)s * a.stride};
      s_slot[u] = s;
    } else if (!pf) {
      const int b = mrank - n_fill;
      a.fills[mrank] = FillEntry{src, a.staging_buf + (size_t)b * a.stride};
      s_slot[u] = -1 - b;
    } else {
      s_slot[u] = INT_MIN;  // prefetch: skipped
    }
  }
  if (u < n && !valid) s_slot[u] = INT_MIN;
  lds_sync();
  for (int p = tid; p < C; p += nt) a.order[p] = ls.order[p];
  if (tid == 0) {
    DevCache* dc = a.cache;
    dc->clock = clock0 + (uint64_t)n_hit + (uint64_t)n_fill;
    if (pf) {
      dc->pf_lookups += (uint64_t)(n_hit + n_miss);
      dc->pf_hits += (uint64_t)n_hit;
      dc->pf_fills += (uint64_t)n_fill;
    } else {
      dc->lookups += (uint64_t)(n_hit + n_miss);
      dc->hits += (uint64_t)n_hit;
      dc->fills += (uint64_t)n_fill;
      dc->bypasses += (uint64_t)(n_miss - n_fill);
    }
    dc->evictions += (uint64_t)ls.evict;
    a.meta->n_fill = pf ? n_fill : n_miss;
    a.meta->n_hit = n_hit;
    a.meta->n_bypass = pf ? 0 : n_miss - n_fill;
  }
  lds_sync();
}

struct FinalizeArgs {
  int T, H, E, k, renorm, has_shared;
  const float* logits;
  int32_t* ids;
  float* gates;
  int32_t* user_ids;
  float* user_gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* inv;
  int32_t* unique;
  int32_t* slotcode;
  int32_t* tok;
  WorkItem* items;
  const uint8_t* shared_w;
  LookupArgs la;
};

template <int NK>
__global__ __launch_bounds__(kFinalizeThreads) void route_finalize_kernel(FinalizeArgs a) {
  __shared__ int s_counts[1024];
  __shared__ unsigned long long s_mask[1024];
  __shared__ int s_offsets[1025];
  __shared__ int s_ids[1024];      // (t, j) -> expert; reused for slot codes
  __shared__ int s_U[1024];
  __shared__ LookupShared ls;
  int* s_slot = s_ids;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int w = tid >> 6, nw = nt >> 6;
  const int T = a.T, E = a.E, k = a.k;

  // Every global load the kernel needs first is issued before the first
  // barrier: the wave's first token's logits and the cache state.
  const TopkArgs ta{a.E, a.k, a.renorm, a.logits, a.ids, a.gates, a.user_ids, a.user_gates};
  uint32_t keys[NK];
  if (w < T) topk_load<NK>(ta, w, keys);
  prefetch_lookup(a.la, ls);
  for (int e = tid; e < 1024; e += nt) {
    s_counts[e] = 0;
    s_mask[e] = 0ull;
  }
  lds_sync();

  // top-k and gates, one wave per token
  for (int t = w; t < T; t += nw) {
    if (t != w) topk_load<NK>(ta, t, keys);
    topk_select<NK>(ta, t, keys, s_ids);
  }
  lds_sync();

  // dispatch: counts, offsets, stable permutation, unique experts
  const int nk = T * k;
  int n_unique;
  for (int f = tid; f < nk; f += nt) {
    const int e = s_ids[f];
    atomicAdd(&s_counts[e], 1);
    atomicOr(&s_mask[e], 1ull << (f / k));
  }
  lds_sync();
  {
    const int e = tid;
    const int cnt = e < E ? s_counts[e] : 0;
    // one scan: offsets in the low 16 bits (T*k <= 1024), unique ranks above
    int both;
    const int ranks = block_excl_scan(cnt | (cnt > 0 ? 1 << 16 : 0), ls.tmp, &both);
    const int off = ranks & 0xFFFF, ur = ranks >> 16;
    const int total = both & 0xFFFF;
    n_unique = both >> 16;
    if (e < E) {
      s_offsets[e] = off;
      a.counts[e] = cnt;
      a.offsets[e] = off;
      if (cnt > 0) {
        s_U[ur] = e;
        a.unique[ur] = e;
      }
    }
    if (tid == 0) {
      s_offsets[E] = total;
      a.offsets[E] = total;
      a.la.meta->n_unique = n_unique;
      a.la.meta->T = T;
    }
  }
  lds_sync();
  for (int f = tid; f < nk; f += nt) {
    const int t = f / k, e = s_ids[f];
    const int rank = __popcll(s_mask[e] & ((1ull << t) - 1ull));
    const int pos = s_offsets[e] + rank;
    a.sorted[pos] = f;
    a.inv[f] = pos;
    a.tok[pos] = t;
  }

  // cache lookup of the unique experts (its first barrier orders the
  // reads of s_ids above before the slot codes overwrite them)
  block_lookup(a.la, ls, s_U, n_unique, s_slot);

  // Work list for the expert kernels: the experts found resident first,
  // then the shared expert, then the experts this call copies (fills and
  // bypasses), each part in ascending expert order.  The expert kernels can
  // then run the first part while the copies are in flight.  One thread per
  // unique expert (n_unique <= 1024 = blockDim.x).
  {
    const int u = tid;
    const int code = u < n_unique ? s_slot[u] : 0;
    const bool resident = u < n_unique && code >= 0 && ls.hit[code];
    const bool copied = u < n_unique && !resident;
    int both;
    const int ranks = block_excl_scan((resident ? 1 : 0) | (copied ? 1 << 16 : 0), ls.tmp, &both);
    const int n_res = both & 0xFFFF;
    const int n_a = n_res + a.has_shared;
    if (u < n_unique) {
      const uint8_t* wptr = code >= 0 ? a.la.slots + (size_t)code * a.la.stride
                                      : a.la.staging_buf + (size_t)(-1 - code) * a.la.stride;
      const int e = s_U[u];
      const int pos = resident ? (ranks & 0xFFFF) : n_a + (ranks >> 16);
      a.items[pos] = WorkItem{wptr, s_offsets[e], s_counts[e]};
      a.slotcode[u] = code;
    }
    if (a.has_shared) {
      for (int t = tid; t < T; t += nt) a.tok[nk + t] = t;
      if (tid == 0) a.items[n_res] = WorkItem{a.shared_w, nk, T};
    }
    if (tid == 0) {
      a.la.meta->n_items = n_unique + a.has_shared;
      a.la.meta->n_items_a = n_a;
      a.la.meta->zero = 0;
    }
  }
}

// Standalone lookup for expert_cache_lookup / expert_cache_fill and the
// prefetch lookup.  The list must be ascending and unique: from the first
// entry that is not above its predecessor on, every entry is passed on as
// invalid (slot code INT_MIN, no state change), so a duplicate can never
// claim two slots or two recency positions.  d_n: the count on the device,
// or NULL for n_max entries; out_slot may be NULL.
__global__ __launch_bounds__(kFinalizeThreads) void cache_lookup_kernel(
    LookupArgs la, const int32_t* experts, const int32_t* d_n, int n_max, int32_t* out_slot) {
  __shared__ int s_U[1024];
  __shared__ int s_slot[1024];
  __shared__ int s_first_bad;
  __shared__ LookupShared ls;
  prefetch_lookup(la, ls);
  int n = d_n ? *d_n : n_max;
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  if (threadIdx.x == 0) s_first_bad = n;
  for (int u = threadIdx.x; u < n; u += blockDim.x) s_U[u] = experts[u];
  lds_sync();
  for (int u = threadIdx.x; u < n; u += blockDim.x)
    if (u > 0 && s_U[u] <= s_U[u - 1]) atomicMin(&s_first_bad, u);
  lds_sync();
  for (int u = threadIdx.x; u < n; u += blockDim.x)
    if (u >= s_first_bad) s_U[u] = -1;
  lds_sync();
  block_lookup(la, ls, s_U, n, s_slot);
  if (out_slot)
    for (int u = threadIdx.x; u < n; u += blockDim.x) out_slot[u] = s_slot[u];
}

LookupArgs make_lookup_args(Ctx* c, int layer, bool insert, FillEntry* fills, DevMeta* meta) {
  LookupArgs la;
  la.layer = layer;
  la.E = c->cfg.n_experts;
  // the lookup runs the same rule on the recency order of the slots the
  // policy lets this layer fill (a layer's share is a contiguous range, and
  // the order of an unresized cache keeps each share's slots in its range)
  la.C = fillable_slots(c, layer, true, &la.slot0);
  la.insert = c->cfg.cache_policy == MOE_CACHE_STATIC ? insert : true;
  la.staging = c->cfg.staging_slots;
  la.key = c->d_key;
  la.stamp = c->d_stamp;
  la.order = c->d_order + la.slot0;
  la.map = c->d_map;
  la.cache = c->d_cache;
  la.pool = c->pool;
  la.slots = c->d_slots;
  la.staging_buf = c->d_staging;
  la.stride = c->stride;
  la.fills = fills;
  la.meta = meta;
  return la;
}

}  // namespace

hipError_t launch_router(const uint16_t* x, int T, int H, int E, const float* wrt,
                         const float* bias, float* logits, hipStream_t st, hipEvent_t ev0,
                         hipEvent_t ev1) {
  if (T <= 1)
    MOE_LAUNCH(router_kernel<1>, E, kRouterWaves * 64, 0, st, ev0, ev1, x, T, H, E, wrt, bias,
               logits);
  else if (T <= 4)
    MOE_LAUNCH(router_kernel<4>, E, kRouterWaves * 64, 0, st, ev0, ev1, x, T, H, E, wrt, bias,
               logits);
  else
    MOE_LAUNCH(router_kernel<kRouterTG>, E, kRouterWaves * 64, 0, st, ev0, ev1, x, T, H, E, wrt,
               bias, logits);
  return hipGetLastError();
}

hipError_t launch_route_finalize(Ctx* c, const DecodeScratch& s, int layer, int T,
                                 int32_t* user_ids, float* user_gates, hipStream_t st,
                                 hipEvent_t ev0, hipEvent_t ev1) {
  FinalizeArgs a;
  a.T = T;
  a.H = c->cfg.hidden;
  a.E = c->cfg.n_experts;
  a.k = c->cfg.top_k;
  a.renorm = c->cfg.renormalize;
  a.has_shared = c->cfg.has_shared;
  a.logits = s.logits;
  a.ids = s.ids;
  a.gates = s.gates;
  a.user_ids = user_ids;
  a.user_gates = user_gates;
  a.counts = s.counts;
  a.offsets = s.offsets;
  a.sorted = s.sorted;
  a.inv = s.inv;
  a.unique = s.unique;
  a.slotcode = s.slotcode;
  a.tok = s.tok;
  a.items = s.items;
  a.shared_w = c->cfg.has_shared ? c->d_shared + (size_t)layer * c->stride : nullptr;
  a.la = make_lookup_args(c, layer, false, s.fills, s.meta);
  const int nk = (a.E + 63) / 64;
  if (nk <= 1)
    MOE_LAUNCH(route_finalize_kernel<1>, 1, kFinalizeThreads, 0, st, ev0, ev1, a);
  else if (nk <= 2)
    MOE_LAUNCH(route_finalize_kernel<2>, 1, kFinalizeThreads, 0, st, ev0, ev1, a);
  else if (nk <= 4)
    MOE_LAUNCH(route_finalize_kernel<4>, 1, kFinalizeThreads, 0, st, ev0, ev1, a);
  else if (nk <= 8)
    MOE_LAUNCH(route_finalize_kernel<8>, 1, kFinalizeThreads, 0, st, ev0, ev1, a);
  else
    MOE_LAUNCH(route_finalize_kernel<16>, 1, kFinalizeThreads, 0, st, ev0, ev1, a);
  return hipGetLastError();
}

hipError_t launch_cache_prefetch(Ctx* c, int layer, const int32_t* d_experts, int n,
                                 const DevMeta* pin, hipStream_t st) {
  LookupArgs la = make_lookup_args(c, layer, true, c->d_pf_fills, c->d_pf_meta);
  la.pin = pin;
  cache_lookup_kernel<<<1, kFinalizeThreads, 0, st>>>(la, d_experts, nullptr, n, nullptr);
  return hipGetLastError();
}

hipError_t launch_cache_lookup(Ctx* c, int layer, const int32_t* d_experts, const int32_t* d_n,
                               int n_max, int32_t* d_slot, bool insert, hipStream_t st) {
  cache_lookup_kernel<<<1, kFinalizeThreads, 0, st>>>(
      make_lookup_args(c, layer, insert, c->ds.fills, c->ds.meta), d_experts, d_n, n_max, d_slot);
  return hipGetLastError();
}

}  // namespace moe
